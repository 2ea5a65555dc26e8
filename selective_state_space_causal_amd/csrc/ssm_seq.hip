// ssm_seq.hip -- one lane per (batch, channel), tokens in order.
//
// The plain form of the channel-local recurrence ("Scaling State-Space Models
// on Multiple GPUs with Tensor Parallelism", euno.news summary of arXiv
// 2602.21144, Methodology item 2): the lane keeps h[0..N) in registers and
// walks its channel's tokens one after another.  It is also the decode step
// (L = 1, resumed from the cache, Methodology item 3).
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

// Per-channel constants held in registers for the whole walk.
template <int NMAX>
struct Channel {
  float w0, w1, w2, w3, cb, dtb, dsk;
  float A2[NMAX];  // A * log2(e): dA = 2^(delta * A2)
};

template <int NMAX, bool EXACT>
__device__ __forceinline__ void load_channel(const ScanArgs& a, int64_t c, Channel<NMAX>& ch) {
  const int N = EXACT ? NMAX : a.N;
  const float* w = a.conv_w + c * 4;
  ch.w0 = w[0];
  ch.w1 = w[1];
  ch.w2 = w[2];
  ch.w3 = w[3];
  ch.cb = a.conv_b ? a.conv_b[c] : 0.0f;
  ch.dtb = a.dt_bias[c];
  ch.dsk = a.Dskip[c];
#pragma unroll
  for (int n = 0; n < NMAX; ++n) ch.A2[n] = (EXACT || n < N) ? a.A[c * N + n] * kLog2e : 0.0f;
}

// One token of one channel: conv window (hist = xi[t-3..t-1]), front end, state update and
// readout.  Returns the gated output in fp32 and shifts the window.
template <typename IO, int NMAX, bool EXACT>
__device__ __forceinline__ float token(const Channel<NMAX>& ch, int N, float (&h)[NMAX], float (&hist)[3],
                                       float xt, float dtr, const IO* Bt, const IO* Ct, const IO* zt) {
  const float v = ch.cb + ch.w0 * hist[0] + ch.w1 * hist[1] + ch.w2 * hist[2] + ch.w3 * xt;
  const float u = silu(v);
  const float delta = softplus(dtr + ch.dtb);
  const float du = delta * u;
  float r = 0.0f;
#pragma unroll
  for (int n = 0; n < NMAX; ++n) {
    if (EXACT || n < N) {
      const float dA = hw_exp2(delta * ch.A2[n]);
      h[n] = fmaf(dA, h[n], du * to_f32(Bt[n]));
      r = fmaf(to_f32(Ct[n]), h[n], r);
    }
  }
  r = fmaf(ch.dsk, u, r);
  if (zt) r *= silu(to_f32(*zt));
  hist[0] = hist[1];
  hist[1] = hist[2];
  hist[2] = xt;
  return r;
}

template <typename IO, int NMAX, bool EXACT>
__global__ __launch_bounds__(256) void prefill_sequential(ScanArgs a) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // flattened (b, c)
  if (row >= a.B * a.D) return;
  const int64_t b = row / a.D, c = row - b * a.D;
  const int N = EXACT ? NMAX : a.N;
  const int64_t L = a.L;            // row stride
  int64_t crow;                     // cache (h / conv) row
  if (!cache_row(a, b, c, crow)) return;
  const int64_t Lb = row_len(a, b);  // tokens to run
  Channel<NMAX> ch;
  load_channel<NMAX, EXACT>(a, c, ch);
  float h[NMAX];
#pragma unroll
  for (int n = 0; n < NMAX; ++n) h[n] = (a.h0 && (EXACT || n < N)) ? a.h0[crow * N + n] : 0.0f;
  float hist[3] = {0.0f, 0.0f, 0.0f};
  if (a.conv0) {
    hist[0] = a.conv0[crow * 3 + 0];
    hist[1] = a.conv0[crow * 3 + 1];
    hist[2] = a.conv0[crow * 3 + 2];
  }
  const IO* x = static_cast<const IO*>(a.x) + row * L;
  const IO* dt = static_cast<const IO*>(a.dt) + row * L;
  const IO* z = a.z ? static_cast<const IO*>(a.z) + row * L : nullptr;
  const IO* Bm = static_cast<const IO*>(a.Bm) + b * L * N;
  const IO* Cm = static_cast<const IO*>(a.Cm) + b * L * N;
  IO* y = static_cast<IO*>(a.y) + row * L;
  for (int64_t t = 0; t < Lb; ++t) {
    const float r = token<IO, NMAX, EXACT>(ch, N, h, hist, to_f32(x[t]), to_f32(dt[t]), Bm + t * N, Cm + t * N,
                                           z ? z + t : nullptr);
    y[t] = from_f32<IO>(r);
  }
#pragma unroll
  for (int n = 0; n < NMAX; ++n)
    if (EXACT || n < N) a.h_out[crow * N + n] = h[n];
  a.conv_out[crow * 3 + 0] = hist[0];
  a.conv_out[crow * 3 + 1] = hist[1];
  a.conv_out[crow * 3 + 2] = hist[2];
}

// Decode step: each lane reads its channel's cache, runs one token and writes the cache back
// in place (the lane owns h[b, c, :] and conv[b, c, :], so no other lane touches them).
template <typename IO, int NMAX, bool EXACT>
__global__ __launch_bounds__(256) void decode_step(ScanArgs a) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= a.B * a.D) return;
  const int64_t b = row / a.D, c = row - b * a.D;
  const int N = EXACT ? NMAX : a.N;
  int64_t crow;  // cache (h / conv) row
  if (!cache_row(a, b, c, crow)) return;
  Channel<NMAX> ch;
  load_channel<NMAX, EXACT>(a, c, ch);
  float h[NMAX];
#pragma unroll
  for (int n = 0; n < NMAX; ++n) h[n] = (EXACT || n < N) ? a.h0[crow * N + n] : 0.0f;
  float hist[3] = {a.conv0[crow * 3 + 0], a.conv0[crow * 3 + 1], a.conv0[crow * 3 + 2]};
  const IO* zt = a.z ? static_cast<const IO*>(a.z) + row : nullptr;
  const float r = token<IO, NMAX, EXACT>(ch, N, h, hist, to_f32(static_cast<const IO*>(a.x)[row]),
                                         to_f32(static_cast<const IO*>(a.dt)[row]),
                                         static_cast<const IO*>(a.Bm) + b * N,
                                         static_cast<const IO*>(a.Cm) + b * N, zt);
  static_cast<IO*>(a.y)[row] = from_f32<IO>(r);
#pragma unroll
  for (int n = 0; n < NMAX; ++n)
    if (EXACT || n < N) a.h_out[crow * N + n] = h[n];
  a.conv_out[crow * 3 + 0] = hist[0];
  a.conv_out[crow * 3 + 1] = hist[1];
  a.conv_out[crow * 3 + 2] = hist[2];
}

static inline dim3 rows_grid(const ScanArgs& a) {
  return dim3((unsigned)((a.B * a.D + 255) / 256));
}

hipError_t launch_sequential(const ScanArgs& a, hipStream_t s) {
  const dim3 grid = rows_grid(a), block(256);
  if (a.bf16) {
    if (a.N == 16) prefill_sequential<bf16_t, 16, true><<<grid, block, 0, s>>>(a);
    else prefill_sequential<bf16_t, 16, false><<<grid, block, 0, s>>>(a);
  } else {
    if (a.N == 16) prefill_sequential<float, 16, true><<<grid, block, 0, s>>>(a);
    else prefill_sequential<float, 16, false><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

bool decode_quad_supported(const ScanArgs& a);
hipError_t launch_decode_quad(const ScanArgs& a, hipStream_t s);

// One launch of the decode step over a.B batch rows (the caller keeps it within the launch
// size limit).
hipError_t launch_decode_rows(const ScanArgs& a, hipStream_t s) {
  if (decode_quad_supported(a)) return launch_decode_quad(a, s);
  const dim3 grid = rows_grid(a), block(256);
  if (a.bf16) {
    if (a.N == 16) decode_step<bf16_t, 16, true><<<grid, block, 0, s>>>(a);
    else decode_step<bf16_t, 16, false><<<grid, block, 0, s>>>(a);
  } else {
    if (a.N == 16) decode_step<float, 16, true><<<grid, block, 0, s>>>(a);
    else decode_step<float, 16, false><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace ssm
