// ssm_gemv.hip -- the projections of include/ssm_proj.h for one token per batch row (a decode
// step): out[b, m] = sum_k W[m, k] * in[b, k] ("Scaling State-Space Models on Multiple GPUs with
// Tensor Parallelism", euno.news summary of arXiv 2602.21144, Methodology items 1 and 3: a
// rank's column / row shard of the mixer's projections, run once per decoded token).
//
// With a single token the product is a matrix-vector one: each weight is used by at most a few
// batch rows, so the call is bound by streaming W from HBM once, not by arithmetic, and a GEMM
// tiling for the matrix cores only adds latency.  Here each wave owns one row of W, eight waves
// to a workgroup; its lanes walk the row in 16-byte pieces (8 bf16 or 4 fp32 weights), 64
// pieces apart, so that the wave reads 1 KiB of contiguous row per load, four loads in flight
// together.  (In the 7B-class layer's decode, in_proj and out_proj with M = 4096, this shape,
// 512 workgroups, made a token 0.5 us faster than two rows per wave in workgroups of four;
// two rows per wave or unrolling by 8 were slower, 16 waves to a workgroup the same.)
// Each piece is multiplied by the same piece of every batch row's input (read through the
// caches: the eight waves of a workgroup share it) with fp32 fused multiply-adds; the 64 lane
// sums of each (row, batch row) are then added across the wave and rounded once to the output
// dtype (bf16: nearest even).  Batch rows are taken up to 8 at a time (W is streamed once per
// group of 8).
#include <stdint.h>

#include "ssm_gemv.h"

namespace ssm {
namespace {

constexpr int kRowsPerWave = 1;
constexpr int kWaves = 8;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;
constexpr int kMaxGroup = 8;  // batch rows per pass over W

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// The E weights or inputs of one 16-byte piece, as fp32.
template <typename IO>
struct Piece;
template <>
struct Piece<uint16_t> {  // bf16
  static constexpr int E = 8;
  __device__ __forceinline__ static void unpack(const u32x4& v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct Piece<float> {
  static constexpr int E = 4;
  __device__ __forceinline__ static void unpack(const u32x4& v, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ void store_out(float v, uint16_t* p) {
  *p = __builtin_bit_cast(uint16_t, (__bf16)v);  // v_cvt_pk_bf16_f32: nearest even
}
__device__ __forceinline__ void store_out(float v, float* p) { *p = v; }

// Batch rows b0 .. b0 + NB - 1; rows of W row0 .. row0 + kRowsPerWave - 1 of this wave (clamped
// into W; only rows below M are stored).
template <typename IO, typename OUT, int NB>
__device__ __forceinline__ void gemv_group(const IO* __restrict__ in, const IO* __restrict__ w, OUT* __restrict__ out,
                                           int K, int M, int b0, int row0) {
  constexpr int E = Piece<IO>::E;
  const int lane = threadIdx.x & 63;
  const int pieces = K / E;
  const u32x4* wr[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int row = row0 + r < M ? row0 + r : M - 1;
    wr[r] = reinterpret_cast<const u32x4*>(w + (int64_t)row * K);
  }
  const u32x4* xr = reinterpret_cast<const u32x4*>(in + (int64_t)b0 * K);
  float acc[kRowsPerWave][NB];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.0f;
#pragma unroll 4
  for (int j = lane; j < pieces; j += 64) {
    u32x4 wv[kRowsPerWave], xv[NB];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) wv[r] = wr[r][j];
#pragma unroll
    for (int b = 0; b < NB; ++b) xv[b] = xr[(int64_t)b * pieces + j];
    float xf[NB][E];
#pragma unroll
    for (int b = 0; b < NB; ++b) Piece<IO>::unpack(xv[b], xf[b]);
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      float wf[E];
      Piece<IO>::unpack(wv[r], wf);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[r][b] = fmaf(wf[e], xf[b][e], acc[r][b]);
    }
  }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float s = wave_sum(acc[r][b]);
      if (lane == 0 && row0 + r < M) store_out(s, out + (int64_t)(b0 + b) * M + row0 + r);
    }
}

template <typename IO, typename OUT>
__global__ __launch_bounds__(64 * kWaves) void gemv_kernel(const IO* __restrict__ in, const IO* __restrict__ w,
                                                         OUT* __restrict__ out, int B, int K, int M) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = blockIdx.x * kRowsPerBlock + wave * kRowsPerWave;
  int b0 = 0;
  for (; B - b0 >= kMaxGroup; b0 += kMaxGroup) gemv_group<IO, OUT, kMaxGroup>(in, w, out, K, M, b0, row0);
  if (B - b0 >= 4) {
    gemv_group<IO, OUT, 4>(in, w, out, K, M, b0, row0);
    b0 += 4;
  }
  if (B - b0 >= 2) {
    gemv_group<IO, OUT, 2>(in, w, out, K, M, b0, row0);
    b0 += 2;
  }
  if (B - b0 >= 1) gemv_group<IO, OUT, 1>(in, w, out, K, M, b0, row0);
}

template <typename IO, typename OUT>
bool launch(const void* in, const void* w, void* out, int B, int K, int M, hipStream_t stream) {
  const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock)), block(64 * kWaves);
  (void)hipGetLastError();
  gemv_kernel<IO, OUT><<<grid, block, 0, stream>>>(static_cast<const IO*>(in), static_cast<const IO*>(w),
                                                  static_cast<OUT*>(out), B, K, M);
  return hipGetLastError() == hipSuccess;
}

}  // namespace

bool gemv_fits(int64_t batch, int64_t in_features, int64_t out_features, bool bf16_io) {
  const int64_t e = bf16_io ? 8 : 4;
  return batch >= 1 && batch <= kGemvMaxBatch && in_features % e == 0 && in_features <= (int64_t)1 << 30 &&
         out_features <= (int64_t)1 << 30 && (out_features + kRowsPerBlock - 1) / kRowsPerBlock <= INT32_MAX;
}

bool gemv(bool bf16_io, bool bf16_out, int64_t batch, int64_t in_features, int64_t out_features, const void* in,
          const void* w, void* out, hipStream_t stream) {
  const int B = (int)batch, K = (int)in_features, M = (int)out_features;
  if (bf16_io)
    return bf16_out ? launch<uint16_t, uint16_t>(in, w, out, B, K, M, stream)
                    : launch<uint16_t, float>(in, w, out, B, K, M, stream);
  return bf16_out ? launch<float, uint16_t>(in, w, out, B, K, M, stream)
                  : launch<float, float>(in, w, out, B, K, M, stream);
}

}  // namespace ssm
