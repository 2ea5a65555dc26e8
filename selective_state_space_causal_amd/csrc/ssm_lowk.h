// ssm_lowk.h -- internal: the projection kernel for a small inner dimension (ssm_lowk.hip), which
// ssm_proj runs for the token-major-in, channel-major-out kinds when it applies.  Not part of the
// C ABI.
#ifndef SSM_LOWK_H
#define SSM_LOWK_H
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// Whether out[b, m, t] = sum_k W[m, k] in[b, t, k] of these sizes runs on this kernel: bf16 in,
// W and out; K a multiple of 16 and at most 256; seqlen a multiple of 8 and at most 2^24; batch x
// seqlen below 2^30.
bool lowk_fits(int64_t batch, int64_t seqlen, int64_t in_features, int64_t out_features, bool bf16_io,
               bool bf16_out);

// Enqueue it (in [batch, seqlen, K], W [M, K], out [batch, M, seqlen], row-major; every pointer
// 16-byte aligned, checked by the caller).  Returns false when the launch fails.
bool lowk(int64_t batch, int64_t seqlen, int64_t in_features, int64_t out_features, const void* in, const void* w,
          void* out, hipStream_t stream);

}  // namespace ssm
#endif  // SSM_LOWK_H
