// ssm_device.h -- device-side helpers shared by the gfx950 kernels of the
// selective state-space scan (io conversions and the per-token front end).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 values travel as raw 16-bit patterns; widening to fp32 is exact.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v.bits << 16); }

template <typename IO>
__device__ __forceinline__ IO from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
// fp32 -> bf16, round to nearest even (finite inputs).
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return bf16_t{(uint16_t)(u >> 16)};
}

// exp2 on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float hw_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// SiLU(v) = v * sigmoid(v) = v / (1 + e^-v).  e^-v overflowing to +inf gives -0 (the limit).
__device__ __forceinline__ float silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + hw_exp2(-v * kLog2e));
}

// softplus(s) = max(s, 0) + log1p(e^-|s|).  log1p(q), q in [0, 1], is ln(u) for u = 1 + q
// rounded, minus the rounding error c = (u - 1) - q (ln(u) - c/u = log1p(q) to first order in
// c, and c/u may be taken as c since |c| <= 2^-24 and the result is about q).  Measured on
// MI355X against fp64 over q in [2^-40, 1]: relative error below 2e-7, so tiny steps keep
// their relative accuracy.  s = -inf gives exactly 0.
__device__ __forceinline__ float softplus(float s) {
  const float q = hw_exp2(-fabsf(s) * kLog2e);
  const float u = 1.0f + q;
  const float c = (u - 1.0f) - q;
  return fmaf(__builtin_amdgcn_logf(u), kLn2, fmaxf(s, 0.0f)) - c;
}

}  // namespace ssm
