// ssm_gemv.h -- internal: the one-token projection kernel (ssm_gemv.hip) that ssm_proj runs for
// seqlen 1.  Not part of the C ABI.
#ifndef SSM_GEMV_H
#define SSM_GEMV_H
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr int64_t kGemvMaxBatch = 16;  // larger batches reuse each weight enough for a GEMM

// Whether out[b, m] = sum_k W[m, k] in[b, k] of these sizes runs as the GEMV: 1 <= batch <= 16,
// in_features a multiple of one 16-byte piece (8 bf16 or 4 fp32) and below 2^30.
bool gemv_fits(int64_t batch, int64_t in_features, int64_t out_features, bool bf16_io);

// Enqueue it (in [batch, K], W [M, K], out [batch, M], row-major; every pointer 16-byte aligned,
// checked by the caller).  Returns false when the launch fails.
bool gemv(bool bf16_io, bool bf16_out, int64_t batch, int64_t in_features, int64_t out_features, const void* in,
          const void* w, void* out, hipStream_t stream);

}  // namespace ssm
#endif  // SSM_GEMV_H
