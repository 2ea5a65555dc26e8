// ssm_conv.hip -- ssm_conv_silu of include/ssm_proj.h: the causal depthwise conv (width 4)
// and SiLU front on its own, u = silu(conv(x)), materialised for the projection that reads
// this slice's channels of u ("Scaling State-Space Models on Multiple GPUs with Tensor
// Parallelism", euno.news summary of arXiv 2602.21144, Methodology item 1: the local mixing
// kernels).
//
// HBM-bound: 2 io values per element (read x, write u).  Each lane owns 8 consecutive tokens
// of one (b, c) row: one 16-byte bf16 load (two for fp32) plus the 3 raw inputs before them,
// taken from the 8 bytes (16 for fp32) just before the lane's tokens, or from conv0 / zeros at
// the row start.  Rows whose length keeps them 16-byte aligned use vector accesses; other
// lengths use element accesses.  Per token the arithmetic is the scan's front end, in the same
// order, so u equals the scan's internal activation before the io rounding.
#include <string.h>

#include "../../include/ssm_proj.h"
#include "ssm_device.h"

namespace ssm {
namespace {

constexpr int EPL = 8;    // tokens per lane
constexpr int TPB = 256;  // threads per workgroup
constexpr int64_t kMaxGrid = int64_t(1) << 20;  // workgroups per launch at most

struct ConvArgs {
  const void* x;
  void* u;
  const float* conv_w;
  const float* conv_b;
  const float* conv0;
  int64_t rows;  // B * D
  int64_t L;
  int64_t D;
  int64_t lanes_per_row;
};

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Lane g of the flattened (row, 8-token group) space.  The lanes of a wave may belong to
// different rows (rows shorter than 512 tokens), so every access is a plain global one with
// its own 64-bit address (a buffer view per row would not be uniform over the wave).
template <typename IO, bool ALIGNED>
__device__ __forceinline__ void conv_lane(const ConvArgs& a, int64_t g) {
  const int64_t row = g / a.lanes_per_row;
  if (row >= a.rows) return;
  const int64_t t0 = (g - row * a.lanes_per_row) * EPL;
  const int64_t c = row % a.D;
  const IO* xr = static_cast<const IO*>(a.x) + row * a.L;

  float xv[EPL + 3];  // xv[0..2] = raw inputs t0-3 .. t0-1, xv[3 + j] = token t0 + j
  if (t0 == 0) {
    for (int j = 0; j < 3; ++j) xv[j] = a.conv0 ? a.conv0[row * 3 + j] : 0.0f;
  }
  if constexpr (ALIGNED) {  // L is a multiple of the 16-byte piece: the lane's tokens are whole pieces
    if constexpr (sizeof(IO) == 2) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(xr + t0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xv[3 + 2 * k] = __uint_as_float(w[k] << 16);
        xv[4 + 2 * k] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
      if (t0 > 0) {  // tokens t0-4 .. t0-1 as one aligned 8-byte load; keep the last three
        const u32x2 h = *reinterpret_cast<const u32x2*>(xr + t0 - 4);
        xv[0] = __uint_as_float(h[0] & 0xFFFF0000u);
        xv[1] = __uint_as_float(h[1] << 16);
        xv[2] = __uint_as_float(h[1] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(xr + t0 + 4 * hh);
#pragma unroll
        for (int k = 0; k < 4; ++k) xv[3 + 4 * hh + k] = __uint_as_float(w[k]);
      }
      if (t0 > 0) {
        const u32x4 h = *reinterpret_cast<const u32x4*>(xr + t0 - 4);
        xv[0] = __uint_as_float(h[1]);
        xv[1] = __uint_as_float(h[2]);
        xv[2] = __uint_as_float(h[3]);
      }
    }
  } else {  // element accesses; tokens past the row end read as zero
#pragma unroll
    for (int j = 0; j < EPL; ++j) xv[3 + j] = t0 + j < a.L ? to_f32(xr[t0 + j]) : 0.0f;
    if (t0 > 0) {
#pragma unroll
      for (int j = 0; j < 3; ++j) xv[j] = to_f32(xr[t0 - 3 + j]);
    }
  }

  const float w0 = a.conv_w[c * 4 + 0], w1 = a.conv_w[c * 4 + 1], w2 = a.conv_w[c * 4 + 2], w3 = a.conv_w[c * 4 + 3];
  const float cb = a.conv_b ? a.conv_b[c] : 0.0f;
  float uv[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const float v = fmaf(w3, xv[3 + j], fmaf(w2, xv[2 + j], fmaf(w1, xv[1 + j], fmaf(w0, xv[j], cb))));
    uv[j] = silu(v);
  }

  const int nvalid = a.L - t0 < EPL ? (int)(a.L - t0) : EPL;
  IO* ur = static_cast<IO*>(a.u) + row * a.L;
  if constexpr (sizeof(IO) == 2) {
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(o[k]) : "v"(uv[2 * k]), "v"(uv[2 * k + 1]));
    if (ALIGNED && nvalid == EPL) {
      *reinterpret_cast<u32x4*>(ur + t0) = u32x4{o[0], o[1], o[2], o[3]};
    } else {
      uint16_t* u16 = reinterpret_cast<uint16_t*>(ur);
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (j < nvalid) u16[t0 + j] = (uint16_t)(o[j >> 1] >> (16 * (j & 1)));
    }
  } else {
    float* uf = reinterpret_cast<float*>(ur);
    if (ALIGNED && nvalid == EPL) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        *reinterpret_cast<float4*>(uf + t0 + 4 * hh) = make_float4(uv[4 * hh], uv[4 * hh + 1], uv[4 * hh + 2], uv[4 * hh + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (j < nvalid) uf[t0 + j] = uv[j];
    }
  }
}

// Grid-stride over lanes, so a launch of any size fits the capped grid (one pass whenever
// the lanes fit in it).
template <typename IO, bool ALIGNED>
__global__ __launch_bounds__(TPB) void conv_silu_kernel(ConvArgs a) {
  const int64_t lanes = a.rows * a.lanes_per_row;
  for (int64_t g = (int64_t)blockIdx.x * TPB + threadIdx.x; g < lanes; g += (int64_t)gridDim.x * TPB)
    conv_lane<IO, ALIGNED>(a, g);
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

}  // namespace
}  // namespace ssm

extern "C" int ssm_conv_silu(const ssm_dims* d, const ssm_params* p, const void* x, const float* conv0, void* u,
                             void* stream) {
  using namespace ssm;
  if (!d || !p || !p->conv_w || !x || !u) return SSM_ERR_NULL;
  if (d->batch < 1 || d->seqlen < 1 || d->d_inner < 1 || d->d_conv != SSM_CONV_WIDTH) return SSM_ERR_SHAPE;
  if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  const int64_t es = d->io_dtype == SSM_BF16 ? 2 : 4;
  int64_t rows, bytes;
  if (__builtin_mul_overflow(d->batch, d->d_inner, &rows) || __builtin_mul_overflow(rows, d->seqlen, &bytes) ||
      __builtin_mul_overflow(bytes, es, &bytes) || d->seqlen * es >= ((int64_t)1 << 31))
    return SSM_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(u, 16) || !aligned(p->conv_w, 16) || (p->conv_b && !aligned(p->conv_b, 4)) ||
      (conv0 && !aligned(conv0, 4)))
    return SSM_ERR_ALIGN;
  if (overlaps(x, bytes, u, bytes)) return SSM_ERR_ALIAS;
  ConvArgs a;
  memset(&a, 0, sizeof a);
  a.x = x;
  a.u = u;
  a.conv_w = p->conv_w;
  a.conv_b = p->conv_b;
  a.conv0 = conv0;
  a.rows = rows;
  a.L = d->seqlen;
  a.D = d->d_inner;
  a.lanes_per_row = (d->seqlen + EPL - 1) / EPL;
  const int64_t threads = rows * a.lanes_per_row, wgs = (threads + TPB - 1) / TPB;
  const dim3 grid((unsigned)(wgs < kMaxGrid ? wgs : kMaxGrid)), tb(TPB);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = d->io_dtype == SSM_BF16;
  const bool al = d->seqlen % (bf ? 8 : 4) == 0;
  if (bf) {
    if (al) conv_silu_kernel<bf16_t, true><<<grid, tb, 0, s>>>(a);
    else conv_silu_kernel<bf16_t, false><<<grid, tb, 0, s>>>(a);
  } else {
    if (al) conv_silu_kernel<float, true><<<grid, tb, 0, s>>>(a);
    else conv_silu_kernel<float, false><<<grid, tb, 0, s>>>(a);
  }
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}
