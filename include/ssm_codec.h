/*
 * ssm_codec.h -- C ABI of the block int8 codec for the tensor-parallel aggregation tensor,
 * on AMD Instinct MI355X (gfx950).  Part of libssm.so, beside the scan of ssm.h.
 *
 * The operation.  Under tensor parallelism each GPU's slice of the mixer ends in a partial
 * output; the ranks' partials are summed by an all-reduce after every token.  "Scaling
 * State-Space Models on Multiple GPUs with Tensor Parallelism" (euno.news summary of arXiv
 * 2602.21144), Methodology item 4 and the Key contributions list: each rank quantizes its
 * tensor to 8 bits before that reduction and dequantizes after it, which cuts the bytes on
 * the interconnect.  The collective itself is not here; these are the two kernels on either
 * side of it: quantize the local partial, and dequantize-and-sum the P parts received.
 *
 * The pages fix no scale granularity or rounding.  This library uses (one reading, stated
 * once here and in the tests' oracle):
 *   - one fp32 scale per block of `block` consecutive elements of the flattened tensor
 *     (the last block may be shorter); block is 32, 64, 128 or 256;
 *   - amax = max |x| over the block; scale s = amax / 127 and multiplier m = 127 / amax,
 *     both correctly rounded fp32 divisions; a block with amax = 0 has s = 0 and codes 0;
 *   - code q = clamp(rint(x * m), -127, 127): one fp32 product, rounded half to even;
 *   - reduce side: y = sum over parts p, in order p = 0, 1, ..., of q_p * s_p, accumulated
 *     in fp32 with fused multiply-adds, then converted to the io dtype (bf16: round to
 *     nearest even).
 *
 * Conventions (as in ssm.h): all tensor pointers are device memory owned by the caller;
 * nothing is allocated or synchronized; work is enqueued on `stream` (a hipStream_t, NULL =
 * the legacy default stream); arguments are validated on the host before any HIP call and
 * an invalid call returns a non-zero ssm_status (ssm.h) and enqueues nothing.  Non-finite
 * inputs are outside the contract.
 */
#ifndef SSM_CODEC_H
#define SSM_CODEC_H

#include <stddef.h>
#include <stdint.h>

#include "ssm.h"

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_Q8_MAX_PARTS 16 /* most parts one ssm_q8_dequant_sum call can sum */

/* Number of scales for n elements: ceil(n / block) (0 for invalid arguments). */
int64_t ssm_q8_num_blocks(int64_t n, int32_t block);

/*
 * Quantize: x [n] io (SSM_F32 or SSM_BF16) -> q [n] int8 and scales [ssm_q8_num_blocks(n,
 * block)] fp32.  Alignment: x 16-byte, q 8-byte, scales 4-byte.  q and scales may not
 * overlap x or each other.  n >= 1.
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE (n < 1, block not 32/64/128/256), SSM_ERR_DTYPE,
 * SSM_ERR_ALIGN, SSM_ERR_ALIAS, SSM_ERR_LAUNCH.
 * Passage: Methodology item 4 of the page cited above (8-bit quantization before the
 * reduction).
 */
int ssm_q8_quantize(int64_t n, int32_t block, int32_t io_dtype, const void* x, int8_t* q, float* scales,
                    void* stream);

/*
 * Dequantize and sum: y [n] io = sum_p q_parts[p][i] * scale_parts[p][i / block], for
 * `parts` received parts (1 <= parts <= SSM_Q8_MAX_PARTS).  q_parts and scale_parts are HOST
 * arrays of `parts` DEVICE pointers, each laid out as ssm_q8_quantize writes them (so the
 * parts may live in separate buffers).  Alignment: every q part 8-byte, every scale part
 * 4-byte, y 16-byte.  y may not overlap any part.
 * Errors: as ssm_q8_quantize, plus SSM_ERR_SHAPE for parts outside [1, SSM_Q8_MAX_PARTS].
 * Passage: Methodology item 4 of the page cited above (dequantization after the reduction).
 */
int ssm_q8_dequant_sum(int64_t n, int32_t block, int32_t io_dtype, int32_t parts, const int8_t* const* q_parts,
                       const float* const* scale_parts, void* y, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SSM_CODEC_H */
