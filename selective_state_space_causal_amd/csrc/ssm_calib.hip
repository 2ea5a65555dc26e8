// ssm_calib.hip -- microbenchmarks of the rates the scan is judged against (include/ssm_calib.h):
// vector-instruction issue (fp32 FMA, the v_exp_f32 transcendental, and a mix of the two) at a
// chosen number of waves per SIMD, and plain HBM copy / read streams.
#include "../../include/ssm_calib.h"
#include <hip/hip_runtime.h>

namespace {

constexpr int kThreads = 256;  // 4 waves: one per SIMD of a CU
constexpr int kChains = 8;     // independent chains per lane
constexpr int kUnroll = 4;     // iterations of the mix per loop trip

constexpr float kM = 0.9990234375f, kC = 0.0009765625f;  // a = a * kM + kC stays in (0, 1]

// Operands that must live in VGPRs (derived from the lane, so the compiler cannot fold them
// into literals or SGPRs).
struct Vops {
  float m, c, x, y;
  __device__ Vops() {
    const float l = 1e-9f * (float)threadIdx.x;
    m = 0.9999999f - l;  // a * m decays by ~1% over the longest runs
    c = kC + l;
    x = 1e-3f + l;       // a += x * y grows by ~10 over the longest runs
    y = 0.5f + l;
  }
};

template <int KIND>
__device__ __forceinline__ float step(float a, const Vops& v) {
  if constexpr (KIND == SSM_CALIB_FMA) {
    return fmaf(a, kM, kC);
  } else if constexpr (KIND == SSM_CALIB_EXP) {
    return __builtin_amdgcn_exp2f(-a);  // converges to the fixed point of 2^-a (~0.641)
  } else if constexpr (KIND == SSM_CALIB_MIX) {
    a = fmaf(a, kM, kC);
    a = fmaf(a, kM, kC);
    a = fmaf(a, kM, kC);
    a = fmaf(a, kM, kC);
    return __builtin_amdgcn_exp2f(-a);
  } else if constexpr (KIND == SSM_CALIB_MUL) {
    return a * v.m;
  } else if constexpr (KIND == SSM_CALIB_FMAC) {
    return fmaf(v.x, v.y, a);
  } else if constexpr (KIND == SSM_CALIB_FMA3) {
    return fmaf(a, v.m, v.c);
  } else {
    static_assert(KIND == SSM_CALIB_DPP, "mix");
    // a += x[lane - 1] * y (lane 0 of each row reads nothing and keeps a); x is never written.
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_shr:1 row_mask:0xf bank_mask:0xf" : "+v"(a) : "v"(v.x), "v"(v.y));
    return a;
  }
}

template <int KIND>
__device__ __forceinline__ void run(int32_t iters, float (&a)[kChains], float (&b)[kChains], const Vops& v) {
  for (int32_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int k = 0; k < kChains; ++k) {
        if constexpr (KIND == SSM_CALIB_MIXI) {
          a[k] = fmaf(a[k], kM, kC);
          a[k] = fmaf(a[k], kM, kC);
          a[k] = fmaf(a[k], kM, kC);
          a[k] = fmaf(a[k], kM, kC);
          b[k] = __builtin_amdgcn_exp2f(-b[k]);
        } else {
          a[k] = step<KIND>(a[k], v);
        }
      }
    }
  }
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void issue_rate(int32_t iters, int64_t split, uint64_t* stamps, float* sink) {
  float a[kChains], b[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) {
    a[k] = 0.25f + 0.01f * (float)k + 1e-6f * (float)threadIdx.x;
    b[k] = 0.5f + 0.01f * (float)k;
  }
  const Vops v;
  // A DPP source needs two wait states after the VALU write that made it; x and y are written
  // here once and only read afterwards.
  if constexpr (KIND == SSM_CALIB_DPP) asm volatile("s_nop 1" ::"v"(v.x), "v"(v.y));
  const int ran = KIND == SSM_CALIB_SPLIT ? ((int64_t)blockIdx.x < split ? SSM_CALIB_FMA : SSM_CALIB_EXP) : KIND;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  if constexpr (KIND == SSM_CALIB_SPLIT) {
    if (ran == SSM_CALIB_FMA) run<SSM_CALIB_FMA>(iters, a, b, v);
    else run<SSM_CALIB_EXP>(iters, a, b, v);
  } else {
    run<KIND>(iters, a, b, v);
  }
  // The chains feed the end stamps, so the stamps cannot be taken before the work is done.
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += a[k] + (KIND == SSM_CALIB_MIXI ? b[k] : 0.0f);
  asm volatile("" ::"v"(s));
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  uint32_t hw, xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  sink[gid] = s;
  if ((threadIdx.x & 63) == 0) {
    uint64_t* w = stamps + (gid >> 6) * SSM_CALIB_STAMP_WORDS;
    w[0] = t0;
    w[1] = t1;
    w[2] = r0;
    w[3] = r1;
    w[4] = hw;
    w[5] = xcc;
    w[6] = (uint64_t)ran;
    w[7] = 0;
  }
}

constexpr int kStreamGrid = 8192;  // workgroups of the copy / read streams (grid-stride)

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void copy_stream(const u32x4* src, u32x4* dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)kStreamGrid * kThreads)
    dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void read_stream(const u32x4* src, int64_t n, float* sink) {
  __shared__ float part[kThreads];
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)kStreamGrid * kThreads) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  part[threadIdx.x] = (float)(acc & 0xFFFF);
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

ssm_status ssm_calib_issue(int kind, int64_t workgroups, int32_t iters, int64_t split, uint64_t* stamps,
                           float* sink, void* stream) {
  if (!stamps || !sink) return SSM_ERR_NULL;
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || kind < SSM_CALIB_FMA || kind > SSM_CALIB_MIXI)
    return SSM_ERR_SHAPE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)workgroups), block(kThreads);
  switch (kind) {
    case SSM_CALIB_FMA: issue_rate<SSM_CALIB_FMA><<<grid, block, 0, s>>>(iters, split, stamps, sink); break;
    case SSM_CALIB_EXP: issue_rate<SSM_CALIB_EXP><<<grid, block, 0, s>>>(iters, split, stamps, sink); break;
    case SSM_CALIB_MIX: issue_rate<SSM_CALIB_MIX><<<grid, block, 0, s>>>(iters, split, stamps, sink); break;
    case SSM_CALIB_MUL: issue_rate<SSM_CALIB_MUL><<<grid, block, 0, s>>>(iters, split, stamps, sink); break;
    case SSM_CALIB_FMAC: issue_rate<SSM_CALIB_FMAC><<<grid, block, 0, s>>>(iters, split, stamps, sink); break;
    case SSM_CALIB_FMA3: issue_rate<SSM_CALIB_FMA3><<<grid, block, 0, s>>>(iters, split, stamps, sink); break;
    case SSM_CALIB_DPP: issue_rate<SSM_CALIB_DPP><<<grid, block, 0, s>>>(iters, split, stamps, sink); break;
    case SSM_CALIB_SPLIT: issue_rate<SSM_CALIB_SPLIT><<<grid, block, 0, s>>>(iters, split, stamps, sink); break;
    default: issue_rate<SSM_CALIB_MIXI><<<grid, block, 0, s>>>(iters, split, stamps, sink); break;
  }
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

ssm_status ssm_calib_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return SSM_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return SSM_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return SSM_ERR_ALIGN;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return SSM_ERR_ALIAS;
  copy_stream<<<kStreamGrid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), (int64_t)(bytes / 16));
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

ssm_status ssm_calib_read(const void* src, size_t bytes, float* sink, void* stream) {
  if (!src || !sink) return SSM_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return SSM_ERR_SHAPE;
  if (!aligned16(src)) return SSM_ERR_ALIGN;
  read_stream<<<kStreamGrid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(src),
                                                                             (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

size_t ssm_calib_read_sink_floats(void) { return kStreamGrid; }

}  // extern "C"
