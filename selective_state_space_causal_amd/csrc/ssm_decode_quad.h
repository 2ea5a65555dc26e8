// ssm_decode_quad.h -- one decode step of one channel on a quad of lanes (lane q of the quad
// owns states 4q .. 4q+3), shared by the decode-step kernel (ssm_decode.hip) and the fused
// per-token layer stages (ssm_decode_fused.hip), so that both compute the same bits from the
// same inputs.
#pragma once
#include "ssm_device.h"

namespace ssm {

constexpr int QS = 4;  // states per lane

// Every lane of the quad ends with the quad's total: quad_perm [1,0,3,2] then [2,3,0,1].
__device__ __forceinline__ float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  return v;
}

// The token's conv window (x0, x1, x2 = the cached raw inputs, oldest first; xt the new one),
// SiLU, softplus step size from the raw dt input dtr, this lane's four states h updated in
// place with decays exp(delta * A4), and the channel's gated output (the same on every lane of
// the quad): (C . h + dsk * u) * silu(zt) when gate, else without the gate factor.
__device__ __forceinline__ float decode_quad_step(float4 w, float cb, float dtb, float dsk, float4 A4, float x0,
                                                  float x1, float x2, float xt, float dtr, float zt, bool gate,
                                                  const float (&Bq)[QS], const float (&Cq)[QS], float (&h)[QS]) {
  const float v = cb + w.x * x0 + w.y * x1 + w.z * x2 + w.w * xt;
  const float u = silu(v);
  const float delta = softplus(dtr + dtb);
  const float du = delta * u;
  const float Aq[QS] = {A4.x, A4.y, A4.z, A4.w};
  float r = 0.0f;
#pragma unroll
  for (int n = 0; n < QS; ++n) {
    const float dA = hw_exp2(delta * (Aq[n] * kLog2e));
    h[n] = fmaf(dA, h[n], du * Bq[n]);
    r = fmaf(Cq[n], h[n], r);
  }
  // Keep the D-skip and gate inputs out of the caller's store branch: the compiler would
  // otherwise sink their loads into it, after the quad sum, and the step would wait for memory
  // twice.
  asm volatile("" ::"v"(dsk), "v"(zt));
  r = quad_sum(r);
  r = fmaf(dsk, u, r);
  const float gz = silu(zt);
  return r * (gate ? gz : 1.0f);
}

}  // namespace ssm
