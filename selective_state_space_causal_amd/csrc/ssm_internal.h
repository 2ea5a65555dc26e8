// ssm_internal.h -- what the C ABI (ssm_api.hip) hands to the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

// One call's tensors and sizes, already validated by the ABI layer.
// Prefill: x/dt/z/y [B, D, L]; Bm/Cm [B, L, N].  Decode: the same with L = 1,
// and h0 == h_out, conv0 == conv_out (in-place cache update).
struct ScanArgs {
  const void* x;
  const void* dt;
  const void* z;  // nullable: no gate
  const void* Bm;
  const void* Cm;
  const float* A;
  const float* Dskip;
  const float* dt_bias;
  const float* conv_w;
  const float* conv_b;  // nullable: zero bias
  const float* h0;      // nullable: zero state
  const float* conv0;   // nullable: zero history
  void* y;
  float* h_out;
  float* conv_out;
  int64_t B, L, D;
  int N;
  int bf16;        // io dtype: 1 = bf16, 0 = fp32
  int chunk_hint;  // prefill decomposition override (0 = automatic)
  // Serving form (cache pool): nullable.
  const int32_t* seqlens;  // [B] tokens of each batch row to run (clamped to [0, L]); null: all L
  const int32_t* slots;    // [B] cache-pool entry of each batch row; outside [0, pool) skips the row
  int64_t pool;            // entries of the cache pool when slots is set
  // Division by D for indices n < 2^30: n / D = (n * d_magic) >> d_shift (set by the decode
  // launcher; see div_magic).
  uint64_t d_magic;
  int d_shift;
};

// Multiply-shift constants for unsigned division by d (1 <= d <= 2^24) of any n < 2^30: with
// l = ceil(log2 d), m = ceil(2^(30 + l) / d) is below 2^31 + 1 and floor(n m / 2^(30 + l)) =
// floor(n / d), because m = (2^(30 + l) + e) / d with 0 <= e < d <= 2^l, so the excess
// n e / (d 2^(30 + l)) stays below 1 / d (Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994).
inline void div_magic(int64_t d, uint64_t* magic, int* shift) {
  int l = 0;
  while ((int64_t(1) << l) < d) ++l;
  const int s = 30 + l;
  *magic = ((uint64_t(1) << s) + uint64_t(d) - 1) / uint64_t(d);
  *shift = s;
}

// Cache row (h / conv entry) of channel c of batch row b, or false when the row is skipped.
__device__ __forceinline__ bool cache_row(const ScanArgs& a, int64_t b, int64_t c, int64_t& crow) {
  if (!a.slots) {
    crow = b * a.D + c;
    return true;
  }
  const int64_t s = a.slots[b];
  if (s < 0 || s >= a.pool) return false;
  crow = s * a.D + c;
  return true;
}

// Tokens to run for batch row b.
__device__ __forceinline__ int64_t row_len(const ScanArgs& a, int64_t b) {
  if (!a.seqlens) return a.L;
  const int64_t n = a.seqlens[b];
  return n < 0 ? 0 : (n > a.L ? a.L : n);
}

// Prefill decompositions.
// chunk_hint selects one explicitly; 0 lets choose_prefill_variant decide.
enum PrefillVariant : int {
  kSequential = 1,  // one lane per (b, c) channel, tokens in order
  kWindowed = 8,    // one wave per (b, c) channel, 8 tokens per lane, DPP scan across lanes
};

int choose_prefill_variant(const ScanArgs& a);
size_t prefill_workspace_bytes(const ScanArgs& a);
hipError_t launch_prefill(const ScanArgs& a, void* workspace, hipStream_t stream);
hipError_t launch_decode(const ScanArgs& a, hipStream_t stream);

}  // namespace ssm
