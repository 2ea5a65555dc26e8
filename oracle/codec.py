"""Block int8 codec for the tensor-parallel aggregation tensor: plain CPU oracle (numpy).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the GPU library.

What it follows: "Scaling State-Space Models on Multiple GPUs with Tensor Parallelism"
(euno.news summary of arXiv 2602.21144), Methodology item 4 and the Key contributions list:
after each token the ranks' partial outputs are summed by an all-reduce; each rank's tensor
is quantized to 8 bits before that reduction and dequantized after it, which cuts the bytes
on the interconnect.  The collective itself needs a second GPU and is not modelled here;
this is the codec on either side of it.

The pages fix neither the scale granularity, nor the rounding, nor how the parts are
summed.  Readings taken (each is the plainest one the rest of the pages supports):
  * symmetric int8 in [-127, 127], one fp32 scale per block of `block` consecutive
    elements of the flattened tensor (the last block may be shorter);
  * scale s = amax / 127, where amax is the largest |x| in the block; codes
    q = clamp(rint(x * (127 / amax)), -127, 127), round half to even; a block whose amax
    is 0 has s = 0 and q = 0;
  * the reduce side sums P received parts: y = sum_p q_p * s_p.
The integer decision is taken in fp32, the GPU kernel's precision: amax is exact, 127 / amax
and amax / 127 are correctly rounded fp32 divisions, x * (127 / amax) is one correctly
rounded fp32 product, and rint rounds half to even.  The dequantized sum is returned in
fp64: each q * s is exact there and the sum of the parts rounds only at fp64 precision, so
it is the value the GPU's fp32 sum approximates.

Pins: tests/test_codec_oracle.py (exact grids, ties, zero blocks, brute-force nearest
code, ragged tails, block independence, exact sums) with planted mistakes in
tests/test_codec_mutants.py.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

QMAX = 127


def num_blocks(n: int, block: int) -> int:
    """Blocks of `block` elements covering n elements (the last may be partial)."""
    return (n + block - 1) // block


def _blocks(x: np.ndarray, block: int) -> Tuple[np.ndarray, int]:
    """Flattened fp32 copy of x padded with zeros to whole blocks, shaped [nb, block]."""
    flat = np.asarray(x, dtype=np.float32).reshape(-1)
    n = flat.size
    nb = num_blocks(n, block)
    padded = np.zeros(nb * block, dtype=np.float32)
    padded[:n] = flat
    return padded.reshape(nb, block), n


def quantize(x: np.ndarray, block: int) -> Tuple[np.ndarray, np.ndarray]:
    """Codes q (int8, same element count as x) and per-block scales s (fp32, [nb])."""
    xb, n = _blocks(x, block)
    amax = np.abs(xb).max(axis=1)                      # zero padding never raises it
    nonzero = amax > 0
    safe = np.where(nonzero, amax, np.float32(1))
    scale = np.where(nonzero, safe / np.float32(QMAX), np.float32(0)).astype(np.float32)
    inv = (np.float32(QMAX) / safe).astype(np.float32)
    codes = np.rint(xb * inv[:, None])                 # fp32 product, half to even
    codes = np.clip(codes, -QMAX, QMAX)
    codes = np.where(nonzero[:, None], codes, 0)
    return codes.astype(np.int8).reshape(-1)[:n], scale


def dequantize_sum(q: np.ndarray, scales: np.ndarray, block: int) -> np.ndarray:
    """y[i] = sum over parts p of q[p, i] * scales[p, i // block], exactly, in fp64.

    q is [P, n] int8 (one row per received part), scales [P, nb] fp32."""
    q = np.asarray(q)
    scales = np.asarray(scales, dtype=np.float32)
    if q.ndim != 2 or scales.ndim != 2 or q.shape[0] != scales.shape[0]:
        raise ValueError("q must be [P, n] and scales [P, nb]")
    parts, n = q.shape
    if scales.shape[1] != num_blocks(n, block):
        raise ValueError("scales must hold one value per block of each part")
    owner = np.arange(n) // block                      # block of each element
    y = np.zeros(n, dtype=np.float64)
    for p in range(parts):
        y += q[p].astype(np.float64) * scales[p, owner].astype(np.float64)
    return y
