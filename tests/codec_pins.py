"""Independent pins for the int8 block codec oracle (oracle/codec.py), importable by the
pin tests and the mutation tests.  Each check takes a codec module (``quantize``,
``dequantize_sum``) and raises AssertionError when it disagrees with what the definition
and exact arithmetic fix.

None of these reuses the oracle's code: the grids are built from integers times powers of
two (so every product and quotient involved is exact), ties are placed by hand, the
nearest-code check tries all 255 codes per element with Python floats, and the sums are
compared with exact integer arithmetic.
"""
from __future__ import annotations

import numpy as np

QMAX = 127


def _grid_blocks(rng, nblocks, block, scales_pow2):
    """Blocks of integer multiples k * s (|k| <= 127, one |k| = 127 per block)."""
    ks = rng.integers(-QMAX, QMAX + 1, size=(nblocks, block))
    for i in range(nblocks):
        ks[i, rng.integers(0, block)] = QMAX if rng.random() < 0.5 else -QMAX
    x = ks.astype(np.float64) * np.asarray(scales_pow2, dtype=np.float64)[:, None]
    return ks, x.astype(np.float32)


def check_exact_grid(codec):
    """x = k * s with s a power of two and amax = 127 s: codes are k and the scale is s."""
    rng = np.random.default_rng(11)
    for block in (32, 64, 128, 256):
        nb = 5
        s = [2.0 ** e for e in (-7, -3, 0, 2, 5)]
        ks, x = _grid_blocks(rng, nb, block, s)
        q, sc = codec.quantize(x, block)
        assert q.dtype == np.int8 and sc.dtype == np.float32
        assert np.array_equal(q.astype(np.int64), ks.reshape(-1)), f"codes differ (block {block})"
        assert np.array_equal(sc, np.asarray(s, np.float32)), f"scales differ (block {block})"


def check_negative_amax(codec):
    """A block whose largest magnitude is negative: amax is a magnitude, the code is -127."""
    block = 64
    x = np.full(block, 0.25, np.float32)
    x[7] = -8.0
    q, sc = codec.quantize(x, block)
    assert sc[0] == np.float32(8.0) / np.float32(127), sc
    assert q[7] == -QMAX, q[7]
    assert q[0] == 4, q[0]  # 0.25 * 127 / 8 = 3.97 -> 4


def check_ties_to_even(codec):
    """amax = 127 gives scale 1 and multiplier 1: halves round to the even neighbour."""
    block = 32
    x = np.zeros(block, np.float32)
    vals = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, 126.5, -126.5, 0.49999997]
    x[: len(vals)] = vals
    q, sc = codec.quantize(x, block)
    assert sc[0] == np.float32(1.0)
    want = [127, 2, 4, -2, -4, 0, 2, 0, 126, -126, 0]
    assert list(q[: len(vals)].astype(int)) == want, list(q[: len(vals)])


def check_zero_blocks(codec):
    """A block of zeros has scale 0 and codes 0; its neighbours are unaffected."""
    block = 32
    x = np.zeros(3 * block, np.float32)
    x[:block] = np.linspace(-1, 1, block, dtype=np.float32)
    x[2 * block:] = 3.0
    q, sc = codec.quantize(x, block)
    assert sc[1] == 0.0 and np.all(q[block:2 * block] == 0)
    assert sc[0] == np.float32(1.0) / np.float32(127) and sc[2] == np.float32(3.0) / np.float32(127)
    assert np.all(q[2 * block:] == QMAX)


def check_nearest_code(codec):
    """Brute force: each code is the integer in [-127, 127] nearest to x / s (Python floats);
    elements within 1e-4 of a tie are skipped (the fp32 multiplier may round either way)."""
    rng = np.random.default_rng(5)
    block = 64
    x = (rng.standard_normal(8 * block) * np.repeat(10.0 ** rng.uniform(-3, 3, 8), block)).astype(np.float32)
    q, sc = codec.quantize(x, block)
    for i in range(x.size):
        xi = float(x[i])
        blk = x[(i // block) * block:(i // block + 1) * block]
        amax = max(abs(float(v)) for v in blk)
        t = xi * QMAX / amax
        if abs(abs(t - np.floor(t)) - 0.5) < 1e-4:
            continue
        best = min(range(-QMAX, QMAX + 1), key=lambda k: abs(t - k))
        assert int(q[i]) == best, (i, xi, int(q[i]), best)
        assert float(sc[i // block]) == float(np.float32(amax) / np.float32(QMAX))


def check_ragged_tail(codec):
    """The last, shorter block is scaled by its own elements only."""
    block = 128
    n = 3 * block + 37
    rng = np.random.default_rng(9)
    x = rng.standard_normal(n).astype(np.float32)
    x[: 3 * block] *= 100.0
    q, sc = codec.quantize(x, block)
    assert q.size == n and sc.size == 4
    tail_amax = max(abs(float(v)) for v in x[3 * block:])
    assert float(sc[3]) == float(np.float32(tail_amax) / np.float32(QMAX))
    assert np.max(np.abs(q[3 * block:].astype(int))) == QMAX


def check_block_independence(codec):
    """Doubling one block (exact in binary) doubles its scale and changes nothing else."""
    block = 64
    rng = np.random.default_rng(3)
    x = rng.standard_normal(6 * block).astype(np.float32)
    q1, s1 = codec.quantize(x, block)
    y = x.copy()
    y[2 * block:3 * block] *= 2
    q2, s2 = codec.quantize(y, block)
    assert np.array_equal(q1, q2)
    assert s2[2] == 2 * s1[2] and np.array_equal(np.delete(s1, 2), np.delete(s2, 2))


def check_round_trip_bound(codec):
    """One part: |x - q s| <= s / 2 (plus fp32 rounding of s) for every element."""
    rng = np.random.default_rng(4)
    block = 128
    x = (rng.standard_normal(20 * block) * 3).astype(np.float32)
    q, sc = codec.quantize(x, block)
    y = codec.dequantize_sum(q[None, :], sc[None, :], block)
    s = np.repeat(sc.astype(np.float64), block)[: x.size]
    err = np.abs(x.astype(np.float64) - y)
    assert np.all(err <= 0.5 * s * (1 + 1e-4) + 1e-30), float(np.max(err / s))


def check_exact_sums(codec):
    """Sum of parts built on exact grids equals the integer-arithmetic sum exactly."""
    rng = np.random.default_rng(8)
    block, nb, parts = 32, 4, 5
    qs, ss, exact = [], [], np.zeros(nb * block, dtype=object)
    for p in range(parts):
        e = rng.integers(-6, 4, size=nb)
        s = [2.0 ** int(v) for v in e]
        ks, x = _grid_blocks(rng, nb, block, s)
        q, sc = codec.quantize(x, block)
        qs.append(q)
        ss.append(sc)
        for i in range(nb * block):  # k * 2^e as an exact rational with denominator 2^6
            exact[i] += int(ks.reshape(-1)[i]) * int(2 ** (int(e[i // block]) + 6))
    y = codec.dequantize_sum(np.stack(qs), np.stack(ss), block)
    want = np.array([float(v) / 64.0 for v in exact])
    assert np.array_equal(y, want), float(np.max(np.abs(y - want)))


def check_each_part_own_scale(codec):
    """Two parts whose scales differ per block: the sum uses each part's own scales."""
    block = 32
    q = np.zeros((2, 2 * block), np.int8)
    q[0, :] = 1
    q[1, :] = 2
    s = np.array([[1.0, 4.0], [0.5, 8.0]], np.float32)
    y = codec.dequantize_sum(q, s, block)
    assert np.all(y[:block] == 1 * 1.0 + 2 * 0.5) and np.all(y[block:] == 1 * 4.0 + 2 * 8.0), y


ALL_CHECKS = {
    "exact_grid": check_exact_grid,
    "negative_amax": check_negative_amax,
    "ties_to_even": check_ties_to_even,
    "zero_blocks": check_zero_blocks,
    "nearest_code": check_nearest_code,
    "ragged_tail": check_ragged_tail,
    "block_independence": check_block_independence,
    "round_trip_bound": check_round_trip_bound,
    "exact_sums": check_exact_sums,
    "each_part_own_scale": check_each_part_own_scale,
}
