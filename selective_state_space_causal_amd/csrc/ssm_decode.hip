// ssm_decode.hip -- decode step: one new token per batch row, resumed from the cached state
// ("Scaling State-Space Models on Multiple GPUs with Tensor Parallelism", euno.news summary
// of arXiv 2602.21144, Methodology item 3: the state left by prefill is reused token by token).
//
// Four lanes share one (b, c) channel; lane q of the quad owns states 4q .. 4q+3, so each
// lane moves its slice of h with one 16-byte load and one 16-byte store (consecutive lanes,
// consecutive addresses).  Every lane of the quad evaluates the channel's front end (conv
// window, SiLU, softplus, gate) on the same broadcast inputs; the readout C_t . h_t is
// summed over the quad with two DPP adds.  Lane 0 of the quad writes y_t and the shifted
// conv window.  Each quad owns its channel's cache entries, so the in-place update is
// race-free.
#include "ssm_decode_quad.h"
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kDecodeBlock = 256;  // threads per workgroup (the launch below uses exactly this)

template <typename IO>
__global__ __launch_bounds__(kDecodeBlock) void decode_quad(ScanArgs a) {
  // Every argument the step reads, fetched in one batch of scalar loads before any arithmetic.
  // Left to itself the compiler loads the tensor pointers in a second batch after the index
  // arithmetic, and each graph node's arguments come from memory not yet in the scalar cache,
  // so the step waited for two scalar round trips before its first vector load.
  asm volatile("" ::"s"(a.x), "s"(a.dt), "s"(a.z), "s"(a.Bm), "s"(a.Cm), "s"(a.A), "s"(a.Dskip), "s"(a.dt_bias),
               "s"(a.conv_w), "s"(a.conv_b), "s"(a.h0), "s"(a.conv0), "s"(a.y), "s"(a.h_out), "s"(a.conv_out),
               "s"(a.B), "s"(a.D), "s"(a.slots), "s"(a.pool), "s"(a.d_magic), "s"(a.d_shift));
  const int64_t gid = (int64_t)blockIdx.x * kDecodeBlock + threadIdx.x;
  const int64_t rows = a.B * a.D;
  const int64_t row = min(gid >> 2, rows - 1);  // a ragged tail repeats the last channel, writes nothing
  const int q = (int)(gid & 3);
  const int64_t b = (int64_t)(((uint64_t)row * a.d_magic) >> a.d_shift), c = row - b * a.D;
  int64_t crow;  // cache (h / conv) row; a skipped batch row leaves as a whole quad (no DPP partner lost)
  if (!cache_row(a, b, c, crow)) return;
  const bool live = (gid >> 2) < rows;

  const float4 w = *reinterpret_cast<const float4*>(a.conv_w + c * 4);
  const float cb = a.conv_b ? a.conv_b[c] : 0.0f;
  const float dtb = a.dt_bias[c], dsk = a.Dskip[c];
  const float4 A4 = *reinterpret_cast<const float4*>(a.A + c * 16 + q * QS);
  const float4 h4 = *reinterpret_cast<const float4*>(a.h0 + crow * 16 + q * QS);
  const float* cv = a.conv0 + crow * 3;
  const float x0 = cv[0], x1 = cv[1], x2 = cv[2];
  const IO* Bt = static_cast<const IO*>(a.Bm) + b * 16 + q * QS;
  const IO* Ct = static_cast<const IO*>(a.Cm) + b * 16 + q * QS;
  const float xt = to_f32(static_cast<const IO*>(a.x)[row]);
  const float dtr = to_f32(static_cast<const IO*>(a.dt)[row]);
  // z is read with the other inputs (x stands in when there is no gate) and the gate applied as
  // a select, so the step waits for one memory round trip, not a second one for z at the end.
  const float zt = to_f32(static_cast<const IO*>(a.z ? a.z : a.x)[row]);

  const float Bq[QS] = {to_f32(Bt[0]), to_f32(Bt[1]), to_f32(Bt[2]), to_f32(Bt[3])};
  const float Cq[QS] = {to_f32(Ct[0]), to_f32(Ct[1]), to_f32(Ct[2]), to_f32(Ct[3])};
  float h[QS] = {h4.x, h4.y, h4.z, h4.w};
  const float r = decode_quad_step(w, cb, dtb, dsk, A4, x0, x1, x2, xt, dtr, zt, a.z != nullptr, Bq, Cq, h);
  if (!live) return;
  *reinterpret_cast<float4*>(a.h_out + crow * 16 + q * QS) = make_float4(h[0], h[1], h[2], h[3]);
  if (q == 0) {
    static_cast<IO*>(a.y)[row] = from_f32<IO>(r);
    float* co = a.conv_out + crow * 3;
    co[0] = x1;
    co[1] = x2;
    co[2] = xt;
  }
}

}  // namespace

bool decode_quad_supported(const ScanArgs& a) { return a.N == 16; }

hipError_t launch_decode_quad(const ScanArgs& a_in, hipStream_t s) {
  ScanArgs a = a_in;
  div_magic(a.D, &a.d_magic, &a.d_shift);  // rows per launch stay below 2^30
  const int64_t lanes = a.B * a.D * 4;
  const dim3 grid((unsigned)((lanes + kDecodeBlock - 1) / kDecodeBlock)), block(kDecodeBlock);
  if (a.bf16) decode_quad<bf16_t><<<grid, block, 0, s>>>(a);
  else decode_quad<float><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ssm
