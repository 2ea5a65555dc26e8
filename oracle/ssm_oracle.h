/*
 * ssm_oracle.h -- fp64 CPU reference of the selective state-space causal scan.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the oracle that the GPU path is checked
 * against.  It shares no code, header, table or helper with the GPU library,
 * and nothing on the product path may include, link or call it: only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * What it computes (one GPU's channel slice, channels independent):
 *   "Scaling State-Space Models on Multiple GPUs with Tensor Parallelism"
 *   (euno.news summary of arXiv 2602.21144), Methodology item 2: each GPU
 *   keeps its own slice of the hidden state and updates it token by token
 *   with no cross-device exchange; Methodology item 3: the hidden state left
 *   by prefill is cached and decode resumes from it.  The pages do not write
 *   the recurrence; the standard Mamba selective-scan form is used (Gu & Dao,
 *   2023): depthwise causal conv (width 4) + SiLU, softplus step size,
 *   exp(delta*A) decay, Euler input term delta*B*u, readout C.h + D*u and the
 *   SiLU(z) output gate.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   x, dt, z, y : [B, D, L]      (channel-major, time contiguous)
 *   Bm, Cm      : [B, L, N]      (shared by all channels of a batch row)
 *   A           : [D, N]         Dskip, dt_bias, conv_b : [D]   conv_w : [D, 4]
 *   h0, h_out   : [B, D, N]      conv0, conv_out : [B, D, 3] (raw inputs, oldest first)
 */
#ifndef SSM_ORACLE_H
#define SSM_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* Conv window (the depthwise causal conv width).  The oracle supports only 4. */
#define SSM_ORACLE_CONV_W 4

/*
 * Run the scan over L tokens for every (b, c) pair.
 *  z        may be NULL: no output gate.
 *  conv_b   may be NULL: zero conv bias.
 *  h0/conv0 may be NULL: start from the zero state and zero conv history
 *           (a fresh prefill).  Non-NULL: resume from that cached state
 *           (a decode step is L = 1 with h0 = h_out, conv0 = conv_out).
 *  h_out/conv_out may alias h0/conv0 (each channel reads its cache fully
 *           before writing it back).
 *  nthreads <= 1 runs single-threaded; otherwise channels are split over
 *           that many POSIX threads (each channel is still sequential in t).
 * Returns 0 on success, -1 on invalid sizes or a NULL required pointer.
 */
int ssm_oracle_scan(int64_t B, int64_t L, int64_t D, int64_t N,
                    const double* x, const double* dt, const double* z,
                    const double* Bm, const double* Cm,
                    const double* A, const double* Dskip, const double* dt_bias,
                    const double* conv_w, const double* conv_b,
                    const double* h0, const double* conv0,
                    double* y, double* h_out, double* conv_out,
                    int nthreads);

#ifdef __cplusplus
}
#endif
#endif
