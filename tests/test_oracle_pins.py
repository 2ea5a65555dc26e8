"""The oracle checked against what the mathematics fixes (no GPU)."""
import itertools

import numpy as np
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("name", sorted(P.ALL_CHECKS))
def test_pin(name):
    P.ALL_CHECKS[name](oracle.scan)


@pytest.mark.parametrize("B,L,D,N", list(itertools.product((1, 2), (1, 2, 3, 4, 5, 64), (1, 3, 16), (1, 4, 16)))[::3])
def test_brute_force_sweep(B, L, D, N):
    for resume in (False, True):
        P.check_brute_force(oracle.scan, B=B, L=L, D=D, N=N, seed=B * 1000 + L * 10 + D + N, resume=resume)


def test_tiny_workload_brute_force():
    """The tiny fp32 workload (batch 1, L=64, 16 channels, 4 states) against the brute force."""
    from selective_state_space_causal_amd import inputs as I
    w = I.WORKLOADS["tiny"]
    prm = I.make_params(w.d_inner, w.d_state)
    seq = I.make_sequence(w.batch, w.seqlen, w.d_inner, w.d_state, w.io)
    f = lambda t: t.double().numpy()
    p = {k: f(seq[k]) for k in ("x", "dt", "z", "Bm", "Cm")}
    p.update({k: f(prm[k]) for k in ("A", "Dskip", "dt_bias", "conv_w", "conv_b")})
    p["h0"] = p["conv0"] = None
    y, h, c = oracle.prefill(seq, prm)
    yb, hb, cb = P.brute_force(p)
    P.close(y, yb)
    P.close(h, hb)
    assert np.array_equal(c, cb)


def test_threads_do_not_change_results():
    p = P.rand_problem(3, 40, 9, 16, 11, resume=True)
    a = P.call(lambda *a, **k: oracle.scan(*a, **k, nthreads=1), p)
    b = P.call(lambda *a, **k: oracle.scan(*a, **k, nthreads=5), p)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_sampled_channels_equal_full_run():
    from selective_state_space_causal_amd import inputs as I
    prm = I.make_params(24, 16)
    seq = I.make_sequence(2, 33, 24, 16, "bf16")
    y, h, c = oracle.prefill(seq, prm)
    pairs = [(0, 0), (1, 23), (0, 17)]
    for (b, ch), (ys, hs, cs) in zip(pairs, oracle.scan_channels(seq, prm, pairs)):
        assert np.array_equal(ys, y[b, ch]) and np.array_equal(hs, h[b, ch]) and np.array_equal(cs, c[b, ch])


def test_rejects_bad_sizes():
    with pytest.raises(ValueError):
        oracle.scan(np.zeros((1, 2, 3)), np.zeros((1, 2, 4)), None, np.zeros((1, 3, 1)), np.zeros((1, 3, 1)),
                    np.zeros((2, 1)), np.zeros(2), np.zeros(2), np.zeros((2, 4)))
