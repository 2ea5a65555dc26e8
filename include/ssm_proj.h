/*
 * ssm_proj.h -- C ABI of the channel-sliced projections on either side of the scan, and of
 * the conv front on its own, on AMD Instinct MI355X (gfx950).  Part of libssm.so.
 *
 * The operation.  "Scaling State-Space Models on Multiple GPUs with Tensor Parallelism"
 * (euno.news summary of arXiv 2602.21144), Methodology item 1: the mixer's packed weight
 * tensor (long-range projections and local mixing kernels) is split across GPUs along the
 * feature dimension, as Transformer tensor parallelism splits its matrices, while item 2 keeps
 * the token-by-token recurrence on each GPU.  A GPU holding channels [c0, c0 + D) of the
 * mixer therefore runs, around the scan of ssm.h:
 *   in_proj   its column shard of the input projection: hidden -> its x and z channels;
 *   conv      the causal conv + SiLU front alone, u = silu(conv(x)), the input of x_proj;
 *   x_proj    the rows of the projection that reads its channels of u and makes the
 *             low-rank step input, B and C: a partial sum over channels, which the ranks add;
 *   dt_proj   the step-size projection of its own channels;
 *   out_proj  its row shard of the output projection: a partial sum, which the ranks add
 *             (the quantized all-reduce of ssm_codec.h).
 * The pages do not write these maps; this library uses the Mamba mixer's (Gu & Dao, 2023).
 *
 * The four projections are dense contractions and run as bf16 (or fp32) GEMMs with fp32
 * accumulation on the matrix cores through hipBLASLt (a plain library GEMM, no fusion);
 * this library supplies the layouts, so that each projection reads and writes the scan's
 * tensors in place:
 *   kind SSM_PROJ_IN / SSM_PROJ_DT (token-major in, channel-major out):
 *       out[b, m, t] = sum_k W[m, k] * in[b, t, k]     in [B, L, K], W [M, K], out [B, M, L]
 *   kind SSM_PROJ_X / SSM_PROJ_OUT (channel-major in, token-major out):
 *       out[b, t, m] = sum_k W[m, k] * in[b, k, t]     in [B, K, L], W [M, K], out [B, L, M]
 * (B = batch, L = seqlen, K = in_features, M = out_features; every tensor row-major and
 * contiguous.)  in_proj is called once for x (W = the x rows) and once for z; x_proj once per
 * output group (low-rank step input, B, C) so that each lands in its own contiguous tensor.
 * With one token per batch row (seqlen 1, a decode step), batch <= 16 and K a multiple of 8
 * (bf16) or 4 (fp32), both layouts are out[b, m] = sum_k W[m, k] in[b, k]: a matrix-vector
 * product bound by reading W from HBM, which runs as a hand-written streaming kernel (fp32
 * fused multiply-adds, W read once per 8 batch rows) instead of a GEMM.  The token-major-in,
 * channel-major-out kinds (SSM_PROJ_IN, SSM_PROJ_DT) with bf16 in and out, K a multiple of 16 up
 * to 256 (the step-size projection, K = its rank), seqlen a multiple of 8 up to 2^24 and
 * batch x seqlen below 2^30 are bound by writing the output; they run as a hand-written kernel
 * (the weights of 64 channels held in each wave's registers, 64-token tiles of the input shared
 * through LDS, fp32 products on the matrix cores, the output rounded to bf16 once).
 *
 * Algorithm choice: hipBLASLt's heuristic offers up to 8 algorithms per shape; for a shape of at
 * least 1e10 flops the first ssm_proj call outside graph capture times each of them on the
 * caller's buffers (two runs each, the host waiting on events) and the context keeps the fastest,
 * so that call is slower and synchronous; later calls of the shape run the kept algorithm only.
 *
 * Conventions (as in ssm.h): device pointers owned by the caller; calls are stream-ordered
 * and asynchronous (but for the first call of a large shape, above); arguments are validated on the host first, and an invalid call returns a
 * non-zero ssm_status and enqueues nothing.  A projection context holds a hipBLASLt handle,
 * created for the device current at ssm_proj_create and valid only on it, and a cache of the
 * algorithm chosen per shape: create one per host thread (a context is not safe for
 * concurrent use).  ssm_proj itself allocates no device memory: its scratch is the caller's
 * workspace (ssm_proj_workspace_bytes); what hipBLASLt sets up inside its handle at creation
 * is hipBLASLt's.
 */
#ifndef SSM_PROJ_H
#define SSM_PROJ_H

#include <stddef.h>
#include <stdint.h>

#include "ssm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ssm_proj_ctx ssm_proj_ctx;

typedef enum { SSM_PROJ_IN = 0, SSM_PROJ_X = 1, SSM_PROJ_DT = 2, SSM_PROJ_OUT = 3 } ssm_proj_kind;

/* Create / destroy a projection context.  create returns SSM_ERR_NULL for a NULL out-pointer
 * and SSM_ERR_LAUNCH when hipBLASLt cannot be initialised. */
int ssm_proj_create(ssm_proj_ctx** ctx);
void ssm_proj_destroy(ssm_proj_ctx* ctx);

/* Device workspace a projection call may use; pass at least this much to ssm_proj. */
size_t ssm_proj_workspace_bytes(void);

/*
 * One projection (layouts above).  io_dtype (SSM_BF16 or SSM_F32) types `in` and `w`;
 * out_dtype types `out` (a partial sum may be kept in fp32).  All sizes >= 1.  Alignment:
 * every pointer 16-byte.  out may not overlap in or w.
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE (a size < 1, a kind out of range, sizes that overflow),
 * SSM_ERR_DTYPE, SSM_ERR_ALIGN, SSM_ERR_ALIAS, SSM_ERR_WORKSPACE (workspace NULL or smaller
 * than ssm_proj_workspace_bytes()), SSM_ERR_LAUNCH (hipBLASLt found no algorithm or failed).
 * Passage: Methodology items 1-2 of the page cited above.
 */
int ssm_proj(ssm_proj_ctx* ctx, int32_t kind, int64_t batch, int64_t seqlen, int64_t in_features,
             int64_t out_features, int32_t io_dtype, int32_t out_dtype, const void* in, const void* w, void* out,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Conv front alone: u[b, c, t] = silu(conv_b[c] + sum_k conv_w[c, k] * xi[b, c, t - 3 + k]),
 * with xi the raw x and xi[-3..-1] = conv0[b, c, 0..2] (NULL = zeros), in the io dtype
 * (bf16: round to nearest even).  The same arithmetic, in the same order, as the front end
 * inside ssm_prefill.  Uses dims (batch, seqlen, d_inner, d_conv = 4, io_dtype) and
 * params->conv_w / conv_b only.  Alignment: x and u 16-byte, conv_w 16-byte, conv_b and conv0
 * 4-byte.  u may not overlap x.
 * Passage: the local mixing kernels of Methodology item 1 of the page cited above.
 */
int ssm_conv_silu(const ssm_dims* dims, const ssm_params* params, const void* x, const float* conv0, void* u,
                  void* stream);

/*
 * Conv front fused into x_proj: lowrank / Bm / Cm = x_proj(u) with u = silu(conv(x)) as in
 * ssm_conv_silu (same arithmetic, same bf16 rounding), computed on the fly and never stored.
 *   out[b, t, m] = sum_c w[m, c] * u[b, c, t],   m < rank + 2 * d_state,
 * rows m in [0, rank) -> lowrank [B, L, rank], [rank, rank + N) -> Bm [B, L, N], the last N ->
 * Cm [B, L, N]: the stacked rows of x_proj that read this slice's channels (w [rank + 2N, D],
 * row-major).  bf16 io only (SSM_ERR_DTYPE otherwise); the sums are fp32 (matrix cores) and
 * rounded to bf16 (nearest even) once.  Uses dims (batch, seqlen, d_inner, d_state, d_conv = 4,
 * io_dtype), params->conv_w / conv_b, conv0 as in ssm_conv_silu.
 * Sizes: d_inner and seqlen multiples of 8, seqlen below 2^24, (rank + 2N) * d_inner * 2 bytes
 * below 2 GiB, rank >= 1 (SSM_ERR_SHAPE otherwise).
 * Alignment: x and w 16-byte, conv_w 16-byte, conv_b and conv0 4-byte, outputs 2-byte (outputs
 * 16-byte aligned, with rank and N multiples of 8, are written in 16-byte pieces).
 * Outputs may not overlap the inputs or each other.
 * Passage: Methodology item 1 of the page cited above (the local mixing kernels and the
 * projection weights of one GPU's feature slice).
 */
int ssm_conv_xproj(const ssm_dims* dims, const ssm_params* params, const void* x, const float* conv0, const void* w,
                   int64_t rank, void* lowrank, void* Bm, void* Cm, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SSM_PROJ_H */
