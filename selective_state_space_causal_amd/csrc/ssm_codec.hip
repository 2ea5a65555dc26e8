// ssm_codec.hip -- the block int8 codec of include/ssm_codec.h: quantize the local partial
// of the tensor-parallel aggregation tensor, and dequantize-and-sum the received parts
// ("Scaling State-Space Models on Multiple GPUs with Tensor Parallelism", euno.news summary
// of arXiv 2602.21144, Methodology item 4).
//
// Both kernels stream HBM once: quantize reads the io tensor and writes one byte per
// element plus one fp32 scale per block; dequant-sum reads one byte per element per part
// plus the scales and writes the io tensor.  Each lane owns 8 consecutive elements (one
// 16-byte bf16 load, two fp32 ones), so a block of 32 / 64 / 128 / 256 elements spans
// 4 / 8 / 16 / 32 lanes of one wave: its |x| maximum is reduced in registers with DPP
// (quad swaps, then the half-row and row mirrors) and, for 32 lanes, one ds_swizzle.  A
// workgroup works on tiles of 2048 elements, a whole number of blocks (quantize: one tile per
// workgroup; dequant-sum: a grid-stride loop), and addresses each tile through raw buffer
// descriptors whose range ends at the tensor's end: a lane past the end reads zeros, its
// stores are dropped, and the one lane that straddles the end uses element accesses.
#include <string.h>

#include "../../include/ssm_codec.h"
#include "ssm_device.h"

namespace ssm {
namespace {

constexpr int EPL = 8;           // elements per lane
constexpr int TPB = 256;         // threads per workgroup
constexpr int EPW = EPL * TPB;   // elements per workgroup
constexpr float QMAX = 127.0f;
// Cache-policy operand of a buffer access: non-temporal.  Used for the streams touched once
// (the codes written by quantize, the codes read and the sum written by dequant-sum); it
// measured 3-8% faster on those and slower on quantize's input loads.
constexpr int NT = 2;
constexpr int64_t DEQUANT_MAX_GRID = 4096;  // 16 workgroups per CU
constexpr int64_t QUANT_MAX_GRID = int64_t(1) << 20;  // keeps a launch within 2^28 work-items

struct QuantArgs {
  const void* x;
  int8_t* q;
  float* scales;
  int64_t n;
};

struct DequantArgs {
  const int8_t* q[SSM_Q8_MAX_PARTS];
  const float* s[SSM_Q8_MAX_PARTS];
  void* y;
  int64_t n;
  int parts;
};

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Maximum over the LPB lanes that hold one block (LPB = 4, 8, 16 or 32; all lanes active).
template <int LPB>
__device__ __forceinline__ float block_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false)));  // lane ^ 1
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false)));  // lane ^ 2
  if constexpr (LPB >= 8)  // lane 7 - i within each half row: pairs the two quads
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false)));
  if constexpr (LPB >= 16)  // lane 15 - i within each row: pairs the two half rows
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false)));
  if constexpr (LPB >= 32)  // lane ^ 16 within each 32 (ds_swizzle bit mode: and 0x1f, xor 0x10)
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (0x10 << 10) | 0x1f)));
  return v;
}

// The lane's 8 io values as fp32 (zeros past the end of the descriptor's range).
template <typename IO>
__device__ __forceinline__ void load8(__amdgpu_buffer_rsrc_t r, int first, bool whole, float (&v)[EPL]) {
  if constexpr (sizeof(IO) == 2) {
    if (whole) {
      const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, first * 2, 0, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int k = 0; k < EPL; ++k)
        v[k] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (first + k) * 2, 0, 0) << 16);
    }
  } else {
    if (whole) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, (first + 4 * h) * 4, 0, 0);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[4 * h + k] = __uint_as_float(w[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < EPL; ++k)
        v[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (first + k) * 4, 0, 0));
    }
  }
}

// One workgroup's tile: elements [e0, e0 + EPW) (fewer at the end).
template <typename IO, int BLOCK>
__device__ __forceinline__ void quantize_tile(const QuantArgs& a, int64_t e0) {
  constexpr int LPB = BLOCK / EPL;
  const int64_t left = a.n - e0;
  const int cnt = left < EPW ? (int)left : EPW;  // elements of this workgroup
  const int first = threadIdx.x * EPL;
  const bool whole = first + EPL <= cnt;

  float v[EPL];
  load8<IO>(rsrc(static_cast<const IO*>(a.x) + e0, (int64_t)cnt * sizeof(IO)), first, whole, v);
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < EPL; ++k) amax = fmaxf(amax, fabsf(v[k]));
  amax = block_max<LPB>(amax);
  // Correctly rounded fp32 divisions (no fast-math); an all-zero block gets scale 0, codes 0.
  const float scale = amax > 0.0f ? amax / QMAX : 0.0f;
  const float mult = amax > 0.0f ? QMAX / amax : 0.0f;

  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    const float c = fminf(fmaxf(__builtin_rintf(v[k] * mult), -QMAX), QMAX);  // half to even
    w[k >> 2] |= ((uint32_t)(int)c & 0xFFu) << (8 * (k & 3));
  }
  const auto rq = rsrc(a.q + e0, cnt);
  if (whole) {
    const u32x2 w2 = {w[0], w[1]};
    __builtin_amdgcn_raw_buffer_store_b64(w2, rq, first, 0, NT);
  } else {
#pragma unroll
    for (int k = 0; k < EPL; ++k)
      __builtin_amdgcn_raw_buffer_store_b8((unsigned char)(w[k >> 2] >> (8 * (k & 3))), rq, first + k, 0, 0);
  }
  if (threadIdx.x % LPB == 0 && first < cnt) a.scales[e0 / BLOCK + threadIdx.x / LPB] = scale;
}

// One tile per workgroup; past QUANT_MAX_GRID tiles the workgroups stride over the rest.
template <typename IO, int BLOCK>
__global__ __launch_bounds__(TPB) void q8_quantize(QuantArgs a) {
  for (int64_t e0 = (int64_t)blockIdx.x * EPW; e0 < a.n; e0 += (int64_t)gridDim.x * EPW)
    quantize_tile<IO, BLOCK>(a, e0);
}

// One 2048-element tile of dequant-sum: elements [e0, e0 + 2048) of every part.
template <typename IO, int BLOCK, int LPB>
__device__ __forceinline__ void dequant_tile(const DequantArgs& a, int64_t e0) {
  const int64_t left = a.n - e0;
  const int cnt = left < EPW ? (int)left : EPW;
  const int nbw = (cnt + BLOCK - 1) / BLOCK;  // scales of this workgroup
  const int first = threadIdx.x * EPL;
  const bool whole = first + EPL <= cnt;

  float acc[EPL];
#pragma unroll
  for (int k = 0; k < EPL; ++k) acc[k] = 0.0f;
  for (int p = 0; p < a.parts; ++p) {
    const auto rq = rsrc(a.q[p] + e0, cnt);
    const auto rs = rsrc(a.s[p] + e0 / BLOCK, nbw * 4);
    const float s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (threadIdx.x / LPB) * 4, 0, 0));
    uint32_t w[2];
    if (whole) {
      const u32x2 w2 = __builtin_amdgcn_raw_buffer_load_b64(rq, first, 0, NT);
      w[0] = w2[0];
      w[1] = w2[1];
    } else {
      w[0] = w[1] = 0u;
#pragma unroll
      for (int k = 0; k < EPL; ++k)
        w[k >> 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rq, first + k, 0, 0) << (8 * (k & 3));
    }
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int code = (int)(w[k >> 2] << (24 - 8 * (k & 3))) >> 24;  // sign-extended byte k
      acc[k] = fmaf((float)code, s, acc[k]);
    }
  }

  const auto ry = rsrc(static_cast<IO*>(a.y) + e0, (int64_t)cnt * sizeof(IO));
  if constexpr (sizeof(IO) == 2) {
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(o[k]) : "v"(acc[2 * k]), "v"(acc[2 * k + 1]));
    if (whole) {
      const u32x4 o4 = {o[0], o[1], o[2], o[3]};
      __builtin_amdgcn_raw_buffer_store_b128(o4, ry, first * 2, 0, NT);
    } else {
#pragma unroll
      for (int k = 0; k < EPL; ++k)
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(o[k >> 1] >> (16 * (k & 1))), ry, (first + k) * 2, 0, 0);
    }
  } else {
    if (whole) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 o4 = {__float_as_uint(acc[4 * h]), __float_as_uint(acc[4 * h + 1]),
                          __float_as_uint(acc[4 * h + 2]), __float_as_uint(acc[4 * h + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(o4, ry, (first + 4 * h) * 4, 0, 0);
      }
    } else {
#pragma unroll
      for (int k = 0; k < EPL; ++k) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[k]), ry, (first + k) * 4, 0, 0);
    }
  }
}

// Grid-stride over 2048-element tiles (the grid is capped at DEQUANT_MAX_GRID workgroups):
// measured 7% faster than one tile per workgroup.
template <typename IO, int BLOCK>
__global__ __launch_bounds__(TPB) void q8_dequant_sum(DequantArgs a) {
  constexpr int LPB = BLOCK / EPL;
  for (int64_t e0 = (int64_t)blockIdx.x * EPW; e0 < a.n; e0 += (int64_t)gridDim.x * EPW)
    dequant_tile<IO, BLOCK, LPB>(a, e0);
}

// One instantiation per (io dtype, block size); KERNEL is q8_quantize or q8_dequant_sum,
// launched on GRID workgroups.
#define SSM_Q8_DISPATCH(KERNEL, GRID)                                                  \
  const dim3 grid((unsigned)(GRID)), tb(TPB);                                          \
  const bool bf = io_dtype == SSM_BF16;                                                \
  switch (block) {                                                                     \
    case 32:                                                                           \
      if (bf) KERNEL<bf16_t, 32><<<grid, tb, 0, s>>>(a);                               \
      else KERNEL<float, 32><<<grid, tb, 0, s>>>(a);                                   \
      break;                                                                           \
    case 64:                                                                           \
      if (bf) KERNEL<bf16_t, 64><<<grid, tb, 0, s>>>(a);                               \
      else KERNEL<float, 64><<<grid, tb, 0, s>>>(a);                                   \
      break;                                                                           \
    case 128:                                                                          \
      if (bf) KERNEL<bf16_t, 128><<<grid, tb, 0, s>>>(a);                              \
      else KERNEL<float, 128><<<grid, tb, 0, s>>>(a);                                  \
      break;                                                                           \
    default:                                                                           \
      if (bf) KERNEL<bf16_t, 256><<<grid, tb, 0, s>>>(a);                              \
      else KERNEL<float, 256><<<grid, tb, 0, s>>>(a);                                  \
      break;                                                                           \
  }                                                                                    \
  return hipGetLastError();

hipError_t launch_quantize(int io_dtype, int block, int64_t n, const QuantArgs& a, hipStream_t s) {
  const int64_t tiles = (n + EPW - 1) / EPW;
  SSM_Q8_DISPATCH(q8_quantize, tiles < QUANT_MAX_GRID ? tiles : QUANT_MAX_GRID)
}

hipError_t launch_dequant_sum(int io_dtype, int block, int64_t n, const DequantArgs& a, hipStream_t s) {
  const int64_t tiles = (n + EPW - 1) / EPW;
  const int64_t grid_tiles = tiles < DEQUANT_MAX_GRID ? tiles : DEQUANT_MAX_GRID;
  SSM_Q8_DISPATCH(q8_dequant_sum, grid_tiles)
}
#undef SSM_Q8_DISPATCH

bool valid_block(int32_t block) { return block == 32 || block == 64 || block == 128 || block == 256; }
bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

struct Span {
  uintptr_t lo, hi;
};
Span span(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Span{lo, lo + (uintptr_t)bytes};
}
bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// n, block and dtype checks shared by both entry points; es = io element size.
int check_sizes(int64_t n, int32_t block, int32_t io_dtype, int64_t* es) {
  if (n < 1 || !valid_block(block) || n > ((int64_t)1 << 52)) return SSM_ERR_SHAPE;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  *es = io_dtype == SSM_BF16 ? 2 : 4;
  return SSM_OK;
}

}  // namespace
}  // namespace ssm

extern "C" {

int64_t ssm_q8_num_blocks(int64_t n, int32_t block) {
  if (n < 1 || !ssm::valid_block(block)) return 0;
  return (n + block - 1) / block;
}

int ssm_q8_quantize(int64_t n, int32_t block, int32_t io_dtype, const void* x, int8_t* q, float* scales,
                    void* stream) {
  using namespace ssm;
  if (!x || !q || !scales) return SSM_ERR_NULL;
  int64_t es;
  if (const int st = check_sizes(n, block, io_dtype, &es)) return st;
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(scales, 4)) return SSM_ERR_ALIGN;
  const Span sx = span(x, n * es), sq = span(q, n), ss = span(scales, ssm_q8_num_blocks(n, block) * 4);
  if (overlaps(sx, sq) || overlaps(sx, ss) || overlaps(sq, ss)) return SSM_ERR_ALIAS;
  QuantArgs a;
  memset(&a, 0, sizeof a);
  a.x = x;
  a.q = q;
  a.scales = scales;
  a.n = n;
  return launch_quantize(io_dtype, block, n, a, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SSM_OK
             : SSM_ERR_LAUNCH;
}

int ssm_q8_dequant_sum(int64_t n, int32_t block, int32_t io_dtype, int32_t parts, const int8_t* const* q_parts,
                       const float* const* scale_parts, void* y, void* stream) {
  using namespace ssm;
  if (!q_parts || !scale_parts || !y) return SSM_ERR_NULL;
  int64_t es;
  if (const int st = check_sizes(n, block, io_dtype, &es)) return st;
  if (parts < 1 || parts > SSM_Q8_MAX_PARTS) return SSM_ERR_SHAPE;
  if (!aligned(y, 16)) return SSM_ERR_ALIGN;
  const Span sy = span(y, n * es);
  const int64_t nb = ssm_q8_num_blocks(n, block);
  DequantArgs a;
  memset(&a, 0, sizeof a);
  for (int p = 0; p < parts; ++p) {
    if (!q_parts[p] || !scale_parts[p]) return SSM_ERR_NULL;
    if (!aligned(q_parts[p], 8) || !aligned(scale_parts[p], 4)) return SSM_ERR_ALIGN;
    if (overlaps(sy, span(q_parts[p], n)) || overlaps(sy, span(scale_parts[p], nb * 4))) return SSM_ERR_ALIAS;
    a.q[p] = q_parts[p];
    a.s[p] = scale_parts[p];
  }
  a.y = y;
  a.n = n;
  a.parts = parts;
  return launch_dequant_sum(io_dtype, block, n, a, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SSM_OK
             : SSM_ERR_LAUNCH;
}

}  // extern "C"
