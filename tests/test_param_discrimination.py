"""The GPU parity cases can see which channel's parameters a kernel reads (CPU only).

Channel-local parameters are the heart of the channel-sliced scan ("Scaling State-Space Models
on Multiple GPUs with Tensor Parallelism", euno.news summary of arXiv 2602.21144, Methodology
item 2: each GPU owns a channel slice with its own parameters).  A kernel that read channel 0's
A row, D-skip or conv bias for every channel, or its neighbour's, must fail the GPU parity
tests.  This checks that it would, with no kernel broken on purpose: on every case of
tests/parity_cases.py the oracle is run once with the case's parameters and once per planted
swap of one parameter's rows -- channel 0's row broadcast to every channel, or the rows rolled
by one channel -- and the swap must move the outputs the GPU tests compare (y, h, and the
decode steps' y and h) by many tolerances:

  * on the channel that moves most, by at least 4 tau;
  * where the case has at least 64 (batch row, token) samples per channel, by at least 20 tau on
    the channel that moves most and by at least 3 tau on 95% or more of the channels the swap
    changes (a handful of tokens from a zero state shows little of the A row: the first token's
    state does not depend on it at all).

tau is the parity tolerance of the io dtype: |gpu - ref| <= tau (1 + |ref|).  The GPU's own
error is below tau, so a result off by 3 tau on a channel fails there.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import parity_cases as PC

TAU = {"f32": 1e-4, "bf16": 2e-2}
SWAPS = [(k, how) for k in ("A", "Dskip", "conv_b") for how in ("channel0", "roll1")]


def swapped(prm, key, how):
    v = prm[key]
    w = v[:1].expand_as(v) if how == "channel0" else torch.roll(v, 1, 0)
    return dict(prm, **{key: w.contiguous()})


def changed_channels(prm, key, how):
    v = prm[key].reshape(prm[key].shape[0], -1)
    w = swapped(prm, key, how)[key].reshape(v.shape[0], -1)
    return np.array([not torch.equal(v[c], w[c]) for c in range(v.shape[0])])


def per_channel(outs, refs):
    """Largest |out - ref| / (1 + |ref|) per channel (axis 1 of every array)."""
    e = None
    for o, r in zip(outs, refs):
        o, r = np.asarray(o, np.float64), np.asarray(r, np.float64)
        err = np.abs(o - r) / (1.0 + np.abs(r))
        err = err.max(axis=tuple(i for i in range(err.ndim) if i != 1)) if err.size else np.zeros(r.shape[1])
        e = err if e is None else np.maximum(e, err)
    return e


def check(run, prm, io, samples, skip=(), spread=True, least=20):
    """run(params) -> list of outputs with the channel on axis 1."""
    ref = run(prm)
    tau = TAU[io]
    seen = 0
    for key, how in SWAPS:
        if prm.get(key) is None or key in skip:
            continue
        mask = changed_channels(prm, key, how)
        if not mask.any():
            continue
        seen += 1
        e = per_channel(run(swapped(prm, key, how)), ref)[mask] / tau
        assert e.max() >= (least if samples >= 64 else 4), f"{key} {how}: largest move {e.max():.1f} tau"
        if samples >= 64 and spread:
            frac = float((e >= 3).mean())
            assert frac >= 0.95, f"{key} {how}: only {frac:.0%} of channels move by 3 tau (min {e.min():.2f})"
    return seen


@pytest.mark.parametrize("case", PC.EDGE, ids=str)
def test_edge_cases_discriminate(case):
    B, L, D, N, io, gate, cb = case
    prm, seq = PC.edge_inputs(*case)
    if D == 1:
        pytest.skip("a single channel has no other channel's parameters to read")
    check(lambda p: oracle.prefill(seq, p, gate=gate)[:2], prm, io, B * L)


@pytest.mark.parametrize("case", PC.WINDOWED, ids=str)
def test_windowed_cases_discriminate(case):
    B, L, D, io = case
    prm, seq = PC.windowed_inputs(*case)
    h0, c0 = PC.random_cache(B, D, 16, seed=L, io=io)

    def run(p):
        y, h, _ = oracle.prefill(seq, p)
        yr, hr, _ = oracle.scan(seq["x"], seq["dt"], None, seq["Bm"], seq["Cm"], p["A"], p["Dskip"], p["dt_bias"],
                                p["conv_w"], p["conv_b"], h0=h0.double().numpy(), conv0=c0.double().numpy())
        return [y, h, yr, hr]

    check(run, prm, io, B * L)


@pytest.mark.parametrize("case", PC.DECODE, ids=str)
def test_decode_cases_discriminate(case):
    io, B, D, N = case
    prm, seq, toks = PC.decode_inputs(*case)

    def run(p):
        _, h, c = oracle.prefill(seq, p)
        outs = []
        for tok in toks:
            y, h, c = oracle.decode_step(tok, p, h, c)
            outs += [y, h]
        return outs

    check(run, prm, io, B * PC.DECODE_T)


@pytest.mark.parametrize("c", PC.sweep_cases(), ids=PC.sweep_id)
def test_sweep_cases_discriminate(c):
    if c["D"] == 1:
        pytest.skip("a single channel has no other channel's parameters to read")
    prm, seq, h0, c0, toks = PC.sweep_inputs(c)
    gate = c["gate"]

    def run(p):
        y, h, cv = oracle.scan(seq["x"], seq["dt"], seq["z"] if gate else None, seq["Bm"], seq["Cm"], p["A"],
                               p["Dskip"], p["dt_bias"], p["conv_w"], p["conv_b"],
                               h0=None if h0 is None else h0.double().numpy(),
                               conv0=None if c0 is None else c0.double().numpy())
        outs = [y, h]
        for tok in toks:
            yt, h, cv = oracle.decode_step(tok, p, h, cv, gate=gate)
            outs += [yt, h]
        return outs

    check(run, prm, c["io"], c["B"] * (c["L"] + 3))


@pytest.mark.parametrize("case", PC.POOL, ids=str)
def test_pool_cases_discriminate(case):
    L, N, io, _ = case
    prm, seq = PC.pool_inputs(L, N, io)
    lens = PC.POOL_LENS(L)

    def run(p):
        outs = []
        for b, n in enumerate(lens):
            if n == 0:
                continue
            row = {k: (v[b:b + 1, :, :n] if k in ("x", "dt", "z") else v[b:b + 1, :n]) for k, v in seq.items()}
            y, h, _ = oracle.prefill(row, p)
            outs += [y, h]
        return outs

    check(run, prm, io, sum(lens))


@pytest.mark.parametrize("name", PC.REGIMES)
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_regime_cases_discriminate(name, io):
    """The regimes that fix A for every channel (running sums, memoryless steps) or make it
    (nearly) irrelevant are checked on D-skip and conv bias only: steps of 1e-28 leave every
    state where it was, steps of ~60 decay every state but the few with |A| below ~0.05 to
    nothing, and with x = 0 in bf16 a channel's drive silu(conv_b[c]) is small where conv_b
    is near zero, so its state weighs little against the bf16 tolerance.  The share of channels
    that move is not asked of the regimes: they bend the inputs so that some channels cannot show
    a swap (a drive near zero, or a D-skip term swamped by a state of size ~60), and their largest
    move is asked to reach 10 tau rather than 20."""
    B, L, D, N = 2, 600, 24, 16
    prm, seq = PC.regime(name, PC.regime_params(D, N), PC.I.make_sequence(B, L, D, N, io, seed=17))
    skip = ("A",) if name in ("a_near_zero", "a_huge", "dt_tiny", "dt_huge") or (name, io) == ("x_zero", "bf16") else ()
    assert check(lambda p: oracle.prefill(seq, p)[:2], prm, io, B * L, skip, spread=False, least=10) >= 4
