/*
 * ssm_calib.h -- rate calibration of the GPU the scan runs on (part of libssm.so).
 *
 * The prefill scan is bound by how fast the SIMDs issue vector instructions, not by memory
 * ("Scaling State-Space Models on Multiple GPUs with Tensor Parallelism", euno.news summary of
 * arXiv 2602.21144, Overview: the recurrent path's speed is what the method is about).  Judging
 * it against that ceiling needs the ceiling measured on the chip itself: these entry points run
 * the microbenchmarks that measure it, and the plain copy and read streams that measure what
 * HBM delivers.  They are measurement tools beside the scan, not part of it.
 *
 * All pointers are device memory owned by the caller; calls are stream-ordered and
 * asynchronous; nothing is allocated.  Errors as in ssm.h (ssm_status).
 */
#ifndef SSM_CALIB_H
#define SSM_CALIB_H
#include <stddef.h>
#include <stdint.h>

#include "ssm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Instruction mixes of ssm_calib_issue, each over 8 independent fp32 chains per lane:
 *   SSM_CALIB_FMA    v_fmamk_f32 (a = a * m + c, m a literal) only;
 *   SSM_CALIB_EXP    v_exp_f32 (a = 2^-a) only;
 *   SSM_CALIB_MIX    four FMAs then one exp per chain and iteration, the exp reading the FMAs'
 *                    result (the scan's ratio of plain to transcendental work is about 6 : 1);
 *   SSM_CALIB_MUL    v_mul_f32 with two VGPR sources only;
 *   SSM_CALIB_FMAC   v_fmac_f32 (a += x * y, three VGPRs read) only;
 *   SSM_CALIB_FMA3   v_fma_f32 in the three-source encoding, four distinct VGPRs, only;
 *   SSM_CALIB_DPP    v_fmac_f32 with a DPP row shift on its first source only (written in inline
 *                    asm, after which the compiler puts an s_nop 0 every 8 instructions);
 *   SSM_CALIB_SPLIT  the waves of the first `split` workgroups run FMA, the others EXP, so that
 *                    a SIMD can hold one wave of each (the stamps say which ran which);
 *   SSM_CALIB_MIXI   four FMAs on chains 0-7 and one exp on 8 further chains per iteration, with
 *                    no dependency between the two. */
typedef enum {
  SSM_CALIB_FMA = 0,
  SSM_CALIB_EXP = 1,
  SSM_CALIB_MIX = 2,
  SSM_CALIB_MUL = 3,
  SSM_CALIB_FMAC = 4,
  SSM_CALIB_FMA3 = 5,
  SSM_CALIB_DPP = 6,
  SSM_CALIB_SPLIT = 7,
  SSM_CALIB_MIXI = 8
} ssm_calib_kind;

/* Words ssm_calib_issue writes per wave into `stamps`. */
#define SSM_CALIB_STAMP_WORDS 8

/*
 * Launch `workgroups` workgroups of 256 threads (4 waves, one per SIMD of a CU when the
 * dispatcher spreads them evenly; workgroups = CUs x w aims at w waves per SIMD), each thread
 * running `iters` iterations of `kind` (8 chains, unrolled by 4: 32 instructions of the mix per
 * iteration and chain group).  `split` is the number of leading workgroups that run FMA under
 * SSM_CALIB_SPLIT (ignored otherwise).
 *   stamps  [workgroups * 4 * SSM_CALIB_STAMP_WORDS] uint64, device: per wave, its shader-clock
 *           counter (s_memtime) at start and end, the constant 100 MHz counter (s_memrealtime)
 *           at start and end, the raw HW_ID and XCC_ID registers (which SIMD of which CU of
 *           which XCD ran it), the mix the wave ran, and 0;
 *   sink    [workgroups * 256] float, device: each thread's final values (keeps the chains
 *           live).
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE (workgroups < 1, iters < 1, kind unknown),
 * SSM_ERR_LAUNCH.
 */
ssm_status ssm_calib_issue(int kind, int64_t workgroups, int32_t iters, int64_t split, uint64_t* stamps,
                           float* sink, void* stream);

/*
 * Plain streams for the HBM context figures: ssm_calib_copy copies `bytes` (a multiple of 16,
 * both bases 16-byte aligned) from src to dst with 16-byte loads and stores; ssm_calib_read
 * reads `bytes` and writes one float per workgroup into `sink` ([ssm_calib_read_sink_floats()]
 * floats) so that the loads are not dropped.
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE (bytes 0 or not a multiple of 16), SSM_ERR_ALIGN,
 * SSM_ERR_LAUNCH.
 */
ssm_status ssm_calib_copy(const void* src, void* dst, size_t bytes, void* stream);
ssm_status ssm_calib_read(const void* src, size_t bytes, float* sink, void* stream);
size_t ssm_calib_read_sink_floats(void);

#ifdef __cplusplus
}
#endif
#endif /* SSM_CALIB_H */
