"""Serving forms on the GPU: ragged prompt lengths and a cache pool indexed by slot, against the
oracle row by row (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_causal_amd as ssm
from selective_state_space_causal_amd import inputs as I
from tests import parity_cases as PC
from tests.gpu_common import DEV, TAU, assert_bitwise, assert_close, dev, f64, note

pytestmark = pytest.mark.gpu
SENT_Y, SENT_H, SENT_C = 640.0, -5.0, -6.0   # exactly representable in bf16


def row_oracle(seq, prm, b, n, h0=None, conv0=None):
    """Oracle for batch row b over its first n tokens (n may be 0)."""
    D = seq["x"].shape[1]
    N = prm["A"].shape[1]
    if n == 0:
        h = np.zeros((D, N)) if h0 is None else np.asarray(h0, np.float64)
        c = np.zeros((D, 3)) if conv0 is None else np.asarray(conv0, np.float64)
        return np.zeros((D, 0)), h, c
    y, h, c = oracle.scan(seq["x"][b:b + 1, :, :n], seq["dt"][b:b + 1, :, :n], seq["z"][b:b + 1, :, :n],
                          seq["Bm"][b:b + 1, :n], seq["Cm"][b:b + 1, :n], prm["A"], prm["Dskip"], prm["dt_bias"],
                          prm["conv_w"], prm.get("conv_b"),
                          h0=None if h0 is None else np.asarray(h0)[None],
                          conv0=None if conv0 is None else np.asarray(conv0)[None])
    return y[0], h[0], c[0]


def run_pool_case(L, N, io, hint, seq, prm):
    B, D, S = PC.POOL_B, PC.POOL_D, PC.POOL_S
    lens, slots = PC.POOL_LENS(L), PC.POOL_SLOTS
    s = dev(seq)
    y = torch.full((B, D, L), SENT_Y, dtype=seq["x"].dtype, device=DEV)
    hp = torch.full((S, D, N), SENT_H, device=DEV)
    cp = torch.full((S, D, 3), SENT_C, device=DEV)
    ssm.prefill_pool(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], dev(prm),
                     torch.tensor(slots, dtype=torch.int32, device=DEV), hp, cp,
                     seqlens=torch.tensor(lens, dtype=torch.int32, device=DEV), chunk_hint=hint, y=y)
    torch.cuda.synchronize()
    yh, hh, ch = f64(y), f64(hp), f64(cp)
    for b, (n, sl) in enumerate(zip(lens, slots)):
        if sl < 0:
            assert np.all(yh[b] == SENT_Y), "skipped row: outputs must stay untouched"
            continue
        yr, hr, cr = row_oracle(seq, prm, b, n)
        assert_close(yh[b, :, :n], yr, TAU[io], f"row {b} y")
        assert np.all(yh[b, :, n:] == SENT_Y), f"row {b}: outputs past its length must stay untouched"
        assert_close(hh[sl], hr, TAU[io], f"row {b} h")
        assert_bitwise(ch[sl], cr, f"row {b} conv")
    for e in set(range(S)) - {sl for sl in slots if sl >= 0}:
        assert np.all(hh[e] == SENT_H) and np.all(ch[e] == SENT_C), f"pool entry {e} must stay untouched"


@pytest.mark.parametrize("L,N,io,hint", PC.POOL)
def test_prefill_pool_ragged_lengths_and_slots(L, N, io, hint):
    note(f"prefill_pool L={L} N={N} {io} hint={hint}")
    prm, seq = PC.pool_inputs(L, N, io)
    run_pool_case(L, N, io, hint, seq, prm)


@pytest.mark.parametrize("L,N,io,hint", [(704, 16, "bf16", 0), (701, 16, "bf16", 0), (600, 16, "f32", 0),
                                         (704, 16, "bf16", 1), (300, 8, "bf16", 0)])
def test_prefill_pool_ignores_what_lies_past_a_row(L, N, io, hint):
    """The tensors of a ragged batch hold whatever the caller left past each row's length
    (stale tokens, padding).  Filled there with NaN and +-Inf in x, dt, z, B and C, every row's
    outputs, state and conv window must still match the oracle run on that row's own tokens:
    the windowed kernel's last window covers tokens past the end and must not let them into
    the state."""
    note(f"prefill_pool poisoned padding L={L} N={N} {io} hint={hint}")
    prm, seq = PC.pool_inputs(L, N, io)
    bad = torch.tensor([float("nan"), float("inf"), -float("inf")])
    poisoned = {k: v.clone() for k, v in seq.items()}
    for b, n in enumerate(PC.POOL_LENS(L)):
        for k, v in poisoned.items():
            tail = v[b, :, n:] if k in ("x", "dt", "z") else v[b, n:]
            tail.copy_(bad[torch.arange(tail.numel()) % 3].reshape(tail.shape).to(v.dtype))
    run_pool_case(L, N, io, hint, poisoned, prm)


@pytest.mark.parametrize("N", [16, 4])
def test_chunked_prefill_and_decode_through_pool(N):
    """Two prefill chunks (the second resumed from the pool) with ragged lengths, then decode steps
    with a permuted slot map: every row against the oracle run on its own tokens."""
    B, D, S, L1, L2, T = 3, 36, 5, 256, 200, 6
    prm = I.make_params_distinct(D, N, seed=53)
    s1 = I.make_sequence(B, L1, D, N, "bf16", seed=53)
    s2 = I.make_sequence(B, L2, D, N, "bf16", seed=54)
    n1, n2 = [256, 100, 17], [200, 3, 150]
    slots = torch.tensor([4, 0, 2], dtype=torch.int32, device=DEV)
    hp = torch.zeros(S, D, N, device=DEV)
    cp = torch.zeros(S, D, 3, device=DEV)
    pd = dev(prm)
    for sq, ns, resume in ((s1, n1, False), (s2, n2, True)):
        d = dev(sq)
        ssm.prefill_pool(d["x"], d["dt"], d["z"], d["Bm"], d["Cm"], pd, slots, hp, cp,
                         seqlens=torch.tensor(ns, dtype=torch.int32, device=DEV), resume=resume)
    ref = []
    for b in range(B):
        _, h, c = row_oracle(s1, prm, b, n1[b])
        _, h, c = row_oracle(s2, prm, b, n2[b], h, c)
        ref.append([h, c])
    torch.cuda.synchronize()
    for b in range(B):
        sl = int(slots[b])
        assert_close(hp[sl], ref[b][0], TAU["bf16"], f"row {b} h after two chunks")
        assert_bitwise(cp[sl], ref[b][1], f"row {b} conv after two chunks")
    perm = [2, 0, 1]  # decode batch row r serves request perm[r]
    dslots = slots[perm].contiguous()
    for t in range(T):
        tok = I.make_decode_token(B, D, N, t, "bf16", seed=55)
        td = dev(tok)
        y = ssm.decode_step_pool(td["x"], td["dt"], td["z"], td["Bm"], td["Cm"], pd, dslots, hp, cp)
        yh = f64(y)
        for r, b in enumerate(perm):
            one = {k: v[r:r + 1] for k, v in tok.items()}
            yr, hr, cr = oracle.decode_step(one, prm, ref[b][0][None], ref[b][1][None])
            ref[b] = [hr[0], cr[0]]
            assert_close(yh[r], yr[0], TAU["bf16"], f"decode step {t} row {r}")
    for b in range(B):
        assert_close(hp[int(slots[b])], ref[b][0], TAU["bf16"], f"row {b} h after decode")


def test_decode_pool_with_identity_slots_equals_decode():
    B, D, N = 4, 96, 16
    prm = dev(I.make_params_distinct(D, N, seed=57))
    h = torch.randn(B, D, N, device=DEV)
    c = torch.randn(B, D, 3, device=DEV)
    h2, c2 = h.clone(), c.clone()
    tok = dev(I.make_decode_token(B, D, N, 0, "bf16", seed=57))
    ya = ssm.decode_step(tok["x"], tok["dt"], tok["z"], tok["Bm"], tok["Cm"], prm, h, c)
    yb = ssm.decode_step_pool(tok["x"], tok["dt"], tok["z"], tok["Bm"], tok["Cm"], prm,
                              torch.arange(B, dtype=torch.int32, device=DEV), h2, c2)
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)) and torch.equal(h, h2) and torch.equal(c, c2)
