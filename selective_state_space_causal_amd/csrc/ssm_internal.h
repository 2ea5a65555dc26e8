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
};

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
