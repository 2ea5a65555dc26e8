/*
 * ssm.h -- C ABI of the selective state-space causal scan for one GPU's
 * channel slice on AMD Instinct MI355X (gfx950).
 *
 * The operation.  A selective state-space (Mamba-family) mixer updates, for
 * every channel c of the local slice and every token t, a small hidden state
 * h[c, 0..N) with an input-dependent decay.  "Scaling State-Space Models on
 * Multiple GPUs with Tensor Parallelism" (euno.news summary of arXiv
 * 2602.21144) fixes the two properties this library is built around:
 *   - Methodology item 2: each GPU keeps its own slice of the hidden state
 *     and updates it token by token with no cross-device exchange, so the
 *     update is channel-local and one GPU can run its slice alone;
 *   - Methodology item 3 (and the Key contributions list): the hidden state
 *     left by prefilling a long prompt is cached, and token-by-token decode
 *     resumes from that cache instead of reprocessing the prompt.
 * The pages do not write the recurrence.  This library computes the standard
 * Mamba selective-scan form (Gu & Dao, 2023).  Per channel (b, c), with xi the
 * raw input x[b, c, :] and xi[-3..-1] the conv history:
 *   v_t  = conv_b[c] + sum_{k=0..3} conv_w[c, k] * xi[t - 3 + k]
 *   u_t  = v_t * sigmoid(v_t)                              (SiLU)
 *   d_t  = softplus(dt[b, c, t] + dt_bias[c])              (step size)
 *   h[n] = exp(d_t * A[c, n]) * h[n] + d_t * Bm[b, t, n] * u_t,  n < N
 *   y_t  = (sum_n Cm[b, t, n] * h[n] + Dskip[c] * u_t) * z_t * sigmoid(z_t)
 * (the gate factor is 1 when z is NULL).  h is updated before y_t reads it.
 *
 * Layouts (row-major, contiguous; B = batch, L = seqlen, D = d_inner of this
 * slice, N = d_state, W = d_conv = 4):
 *   x, dt, z, y     [B, D, L]  io dtype (channel-major: one channel's tokens contiguous)
 *   Bm, Cm          [B, L, N]  io dtype (shared by all channels of a batch row)
 *   A               [D, N]     fp32     Dskip, dt_bias, conv_b [D] fp32   conv_w [D, 4] fp32
 *   h  (state)      [B, D, N]  fp32
 *   conv (window)   [B, D, 3]  fp32: the last three RAW inputs xi[L-3..L-1], oldest first
 *                              (zero, or the given history, where L - 3 + j < 0)
 * Decode-step tensors are the L = 1 case: x_t, dt_t, z_t, y_t [B, D]; B_t, C_t [B, N].
 *
 * Conventions shared by every entry point.
 *   Ownership  all tensor pointers are device memory owned by the caller; the
 *              library allocates nothing, frees nothing and keeps no mutable
 *              global state, so it may be called from several host threads.
 *   Ordering   work is enqueued on `stream` (a hipStream_t; NULL = the legacy
 *              default stream) and runs asynchronously; the library never
 *              synchronizes the host with the device.
 *   Errors     arguments are validated on the host before any HIP call; an
 *              invalid call returns a non-zero ssm_status and enqueues nothing.
 *              A launch failure returns SSM_ERR_LAUNCH.  No exception crosses
 *              the ABI.  Non-finite inputs are outside the contract.
 *   Alignment  prefill: every tensor base pointer 16-byte aligned.  Decode step: io
 *              tensors naturally aligned (2 bytes bf16, 4 bytes fp32), h 16-byte, the conv
 *              window 4-byte.  Parameters (both): A and conv_w 16-byte, the rest 4-byte.
 *   Aliasing   outputs may not overlap inputs or each other, except that the
 *              decode step updates h and conv in place by design.
 *   Device     kernels run on the calling thread's current HIP device.
 *   Launches   a call may enqueue several kernel launches: a batch too large for one launch
 *              (more than 2^31 work-items) is split into launches over consecutive batch
 *              rows.  Channels are never split, so the results are the same bits.
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 2
#define SSM_MAX_STATE 16 /* largest supported d_state */
#define SSM_CONV_WIDTH 4 /* the only supported d_conv */
#define SSM_MAX_D_INNER (1 << 24) /* largest d_inner of one call */

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = 1,      /* a required pointer is NULL */
  SSM_ERR_SHAPE = 2,     /* a size is < 1, d_inner > SSM_MAX_D_INNER, d_state > 16, d_conv != 4,
                            or a byte count overflows int64 */
  SSM_ERR_DTYPE = 3,     /* io_dtype is not SSM_F32 or SSM_BF16 */
  SSM_ERR_ALIGN = 4,     /* a tensor base pointer breaks the alignment rule below */
  SSM_ERR_ALIAS = 5,     /* an output overlaps an input or another output */
  SSM_ERR_WORKSPACE = 6, /* workspace NULL or smaller than ssm_prefill_workspace_bytes() */
  SSM_ERR_LAUNCH = 7,    /* a kernel launch failed (hipGetLastError) */
  SSM_ERR_SCRATCH = 8    /* the call needs more scratch than a no-allocation entry point holds
                            (ssm_decode_fused_noalloc: SSM_NOALLOC_SCRATCH_BYTES) */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/* Sizes of one call.  seqlen is ignored by ssm_decode_step. */
typedef struct {
  int64_t batch;    /* B >= 1 */
  int64_t seqlen;   /* L >= 1 */
  int64_t d_inner;  /* D in [1, SSM_MAX_D_INNER]: channels of this GPU's slice */
  int64_t d_state;  /* N in [1, 16] */
  int64_t d_conv;   /* must be 4 */
  int32_t io_dtype; /* ssm_dtype of x, dt, z, Bm, Cm and y */
  int32_t chunk_hint; /* prefill decomposition: 0 = automatic, 1 = one lane per channel walking
                         its tokens in order, 8 = one wave per channel with 8 tokens per lane
                         (d_state 16 only; otherwise the one-lane form runs).  Any other value
                         is SSM_ERR_SHAPE.  The automatic choice of decomposition depends on
                         d_state and L only; the workgroup shape may follow batch * d_inner but
                         never changes a result bit.  So a channel slice or a batch row run
                         alone reproduces the full run bit for bit. */
} ssm_dims;

/* Per-channel parameters, device fp32.  conv_b may be NULL (zero bias). */
typedef struct {
  const float* A;       /* [D, N]  decay rates (A = -exp(A_log) precomputed by the caller) */
  const float* Dskip;   /* [D]     skip weight */
  const float* dt_bias; /* [D]     step-size bias */
  const float* conv_w;  /* [D, 4]  conv_w[c, k] multiplies xi[t - 3 + k] (k = 3 is the current token) */
  const float* conv_b;  /* [D]     conv bias, or NULL */
} ssm_params;

/* ABI version of the loaded library (SSM_ABI_VERSION when it matches this header). */
int ssm_abi_version(void);

/* Static, human-readable name of a status code ("unknown status" for others). */
const char* ssm_status_str(int status);

/* Device workspace in bytes that ssm_prefill needs for these sizes (0 = none).
 * Returns 0 for invalid sizes as well; ssm_prefill then reports the error. */
size_t ssm_prefill_workspace_bytes(const ssm_dims* dims);

/*
 * Prefill: run the recurrence over all L tokens of every (b, c) channel,
 * write y, and leave the state cache for decode:
 *   h_out[b, c, :]    = h after token L - 1
 *   conv_out[b, c, j] = xi[L - 3 + j]   (j = 0, 1, 2)
 * Inputs: x, dt, z (NULL = no gate), Bm, Cm as laid out above.  h0 and conv0
 * (both NULL for a fresh prompt) resume from an earlier cache instead of the
 * zero state and zero history; this is chunked prefill: prefilling L1 tokens
 * and then L2 more from the cache equals prefilling L1 + L2.  h_out and
 * conv_out may not overlap h0 and conv0.
 * workspace: device memory of at least ssm_prefill_workspace_bytes(dims)
 * bytes (NULL allowed when that is 0); its contents need no initialisation
 * and are scratch after the call.
 * Passage: the state-caching method (Methodology item 3) and the channel-
 * local recurrence (Methodology item 2) of the page cited above.
 */
int ssm_prefill(const ssm_dims* dims, const ssm_params* params,
                const void* x, const void* dt, const void* z,
                const void* Bm, const void* Cm,
                const float* h0, const float* conv0,
                void* y, float* h_out, float* conv_out,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode step: one new token per batch row, resumed from the cache.
 *   y_t[b, c]        = output for the token (same formula, L = 1)
 *   h[b, c, :]       <- updated state                          (in place)
 *   conv_state[b, c] <- (conv[1], conv[2], x_t[b, c])          (in place)
 * Inputs x_t, dt_t, z_t (NULL = no gate) [B, D]; B_t, C_t [B, N]; the cache
 * h [B, D, N] and conv_state [B, D, 3] as written by ssm_prefill or by an
 * earlier step.  dims->seqlen and dims->chunk_hint are ignored.
 * Passage: decode reuses the cached state instead of reprocessing the
 * processed tokens (Methodology item 3 of the page cited above).
 */
int ssm_decode_step(const ssm_dims* dims, const ssm_params* params,
                    const void* x_t, const void* dt_t, const void* z_t,
                    const void* B_t, const void* C_t,
                    void* y_t, float* h, float* conv_state, void* stream);

/*
 * Serving forms: ragged batches and a cache pool.  A server keeps one h / conv entry per
 * live request in a pool and runs whichever requests are ready, so batch row b maps to pool
 * entry slots[b], and prefill rows may hold prompts of different lengths padded to L.
 * Passages: state caching between prefill and decode (Methodology item 3 and the Key
 * contributions list of the page cited above) with the batch sizes and context lengths the
 * same page varies (Methodology item 5).
 *
 *   h_pool    [S, D, N] fp32 and conv_pool [S, D, 3] fp32, S = pool_size >= 1
 *   slots     device int32 [B]: pool entry of batch row b; a value outside [0, S) skips row b
 *             entirely (nothing of that row is read from or written to the pool, and its
 *             outputs are left untouched).  Two rows naming the same entry race: undefined.
 *   seqlens   device int32 [B] or NULL: row b runs its first clamp(seqlens[b], 0, L) tokens;
 *             outputs past that length are left untouched.  NULL = L tokens for every row.
 * The other tensors and all conventions are those of ssm_prefill / ssm_decode_step; the
 * pools follow the prefill alignment rule in ssm_prefill_pool and h_pool 16-byte, conv_pool
 * 4-byte, slots 4-byte in ssm_decode_step_pool.
 */

/*
 * Prefill into a cache pool: for every row b with a valid slot, run its first n_b tokens and
 * store the final state in h_pool[slots[b]], the last three raw inputs (before token n_b) in
 * conv_pool[slots[b]].  resume != 0 starts each row from its pool entry (chunked prefill:
 * prompts arrive in pieces); resume == 0 starts from the zero state and zero history.  The
 * pool is read and rewritten in place.  The prefill decomposition is chosen as in
 * ssm_prefill (dims->chunk_hint).
 */
int ssm_prefill_pool(const ssm_dims* dims, const ssm_params* params,
                     const void* x, const void* dt, const void* z,
                     const void* Bm, const void* Cm,
                     const int32_t* seqlens, const int32_t* slots, int64_t pool_size, int resume,
                     void* y, float* h_pool, float* conv_pool, void* stream);

/*
 * Decode step against a cache pool: row b reads and updates h_pool[slots[b]] and
 * conv_pool[slots[b]] in place (rows with an invalid slot are skipped).
 */
int ssm_decode_step_pool(const ssm_dims* dims, const ssm_params* params,
                         const void* x_t, const void* dt_t, const void* z_t,
                         const void* B_t, const void* C_t,
                         const int32_t* slots, int64_t pool_size,
                         void* y_t, float* h_pool, float* conv_pool, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SSM_H */
