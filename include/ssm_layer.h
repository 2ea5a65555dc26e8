/*
 * ssm_layer.h -- the per-token stages of one rank's mixer layer between its two large
 * projections, fused (part of libssm.so).
 *
 * Decoding one token through one rank's slice of a selective-SSM mixer layer ("Scaling
 * State-Space Models on Multiple GPUs with Tensor Parallelism", euno.news summary of arXiv
 * 2602.21144: Methodology item 1 splits the mixer's projections across GPUs by channel,
 * item 3 resumes decode from the state cached at prefill) runs, per batch row:
 *   x_t, z_t  = in_proj (column shard)                          [d_model] -> [D] each
 *   u         = silu(conv(conv cache, x_t))                     the conv front from the cache
 *   r, B_t, C_t = x_proj rows that read these channels, on u    [D] -> [R], [N], [N] (partial sums)
 *   dt        = dt_proj (r)                                     [R] -> [D]
 *   y_t, h, conv = the decode step (ssm_decode_step of ssm.h)   h and conv updated in place
 *   out       = out_proj (row shard)                            [D] -> [d_model] (a partial sum)
 * ssm_decode_fused runs the four middle stages in two kernels instead of one launch each
 * (conv front, x_proj, dt_proj, decode step); the projections either side stay GEMMs
 * (ssm_proj.h).  Every intermediate is rounded to the io dtype at the point where the unfused
 * composition stores it (u, r, B_t, C_t, dt), so the fused and unfused paths compute the same
 * values up to fp32 summation order.  On one GPU the x_proj partial sums are used as they are
 * (their all-reduce across ranks is not part of this library).
 *
 * Layouts (row-major, contiguous; B = batch, D = d_inner of this slice, N = d_state = 16,
 * R = rank of the step-size projection):
 *   x_t, z_t, y_t   [B, D]      io dtype        (z_t may be NULL: no gate)
 *   h               [B, D, N]   fp32, in place  (16-byte aligned)
 *   conv            [B, D, 3]   fp32, in place  (the last three raw inputs, oldest first)
 *   w_x             [R + 2N, D] io dtype: rows 0..R-1 make r, then N rows make B_t, N make C_t
 *   w_dt            [D, R]      io dtype
 *   params          as in ssm.h (A [D, N], Dskip, dt_bias, conv_w [D, 4], conv_b)
 *   workspace       device, ssm_decode_fused_workspace_bytes(): the x_proj partial sums of
 *                   each block of 64 channels, fp32 [B, ceil(D / 64), R + 2N]; every byte read
 *                   is written first in the same call, so it needs no clearing
 * Sizes: d_state must be 16, 1 <= R and R + 2N <= 512; seqlen and chunk_hint of ssm_dims are
 * ignored.  Conventions (ownership, ordering, errors before any HIP call, no allocation, no
 * global state) as in ssm.h; the weights and parameters are inputs and may not overlap an
 * output; h and conv are updated in place by design.
 */
#ifndef SSM_LAYER_H
#define SSM_LAYER_H
#include <stddef.h>
#include <stdint.h>

#include "ssm.h"

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_FUSED_MAX_ROWS 512 /* largest R + 2N of ssm_decode_fused */

/* Bytes of workspace ssm_decode_fused needs for these sizes (0 on invalid sizes). */
size_t ssm_decode_fused_workspace_bytes(const ssm_dims* d, int64_t rank);

/* One decoded token through the conv front, x_proj, dt_proj and the decode step (above).
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE (sizes, d_state != 16, R + 2N > 512), SSM_ERR_DTYPE,
 * SSM_ERR_ALIGN, SSM_ERR_ALIAS, SSM_ERR_WORKSPACE, SSM_ERR_LAUNCH. */
ssm_status ssm_decode_fused(const ssm_dims* d, const ssm_params* p, const void* w_x, const void* w_dt, int64_t rank,
                            const void* x_t, const void* z_t, void* y_t, float* h, float* conv_state,
                            void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): ssm_decode_fused without a workspace argument.  Its
 * scratch is a fixed array of SSM_NOALLOC_SCRATCH_BYTES in the library's device code, one per
 * GPU, held until the process ends; its address is looked up on the first call on each device
 * (with that device current) and kept.  The call allocates nothing.  Every call on one GPU
 * shares that GPU's array, so calls that overlap in time on one GPU (other streams, other host
 * threads) race and must not be made; nothing in the array needs clearing (each call writes
 * every byte it reads).  Sizes whose ssm_decode_fused_workspace_bytes() exceeds
 * SSM_NOALLOC_SCRATCH_BYTES are rejected with SSM_ERR_SCRATCH before any HIP call.  Other
 * arguments, errors and results as ssm_decode_fused (the same kernels). */
#define SSM_NOALLOC_SCRATCH_BYTES (16u << 20)
ssm_status ssm_decode_fused_noalloc(const ssm_dims* d, const ssm_params* p, const void* w_x, const void* w_dt,
                                    int64_t rank, const void* x_t, const void* z_t, void* y_t, float* h,
                                    float* conv_state, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SSM_LAYER_H */
