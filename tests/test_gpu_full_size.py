"""Full-size workloads on the GPU, checked against the oracle on sampled channels (the
recurrence is channel-local, so each sampled (b, c) is computed exactly and alone)."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_causal_amd as ssm
from selective_state_space_causal_amd import inputs as I
from tests.gpu_common import DEV, TAU, assert_bitwise, assert_close, dev, f64, note, sample_pairs

pytestmark = pytest.mark.gpu


def prefill_and_check(name, k=24):
    w = I.WORKLOADS[name]
    note(f"{name}: B={w.batch} L={w.seqlen} D={w.d_inner} N={w.d_state} {w.io}: generating")
    prm = I.make_params(w.d_inner, w.d_state, dt_range=w.dt_range)
    pd = dev(prm)
    s = I.make_sequence_device(w.batch, w.seqlen, w.d_inner, w.d_state, w.io, device=DEV)
    note(f"{name}: prefill")
    y, h, c = ssm.prefill(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], pd)
    torch.cuda.synchronize()
    pairs = sample_pairs(w.batch, w.d_inner, k)
    note(f"{name}: oracle on {len(pairs)} channels")
    ref = oracle.scan_channels(s, prm, pairs)
    for (b, ch), (yr, hr, cr) in zip(pairs, ref):
        assert_close(y[b, ch], yr, TAU[w.io], f"{name} y[{b},{ch}]")
        assert_close(h[b, ch], hr, TAU[w.io], f"{name} h[{b},{ch}]")
        assert_bitwise(c[b, ch], cr, f"{name} conv[{b},{ch}]")
    return w, prm, pd, s, (y, h, c), pairs, ref


def decode_and_check(name, w, prm, pd, h, c, pairs, ref):
    st = {p: (r[1][None, None], r[2][None, None]) for p, r in zip(pairs, ref)}
    note(f"{name}: {w.decode_steps} decode steps")
    for t in range(w.decode_steps):
        tok = I.make_decode_token(w.batch, w.d_inner, w.d_state, t, w.io)
        td = dev(tok)
        y = ssm.decode_step(td["x"], td["dt"], td["z"], td["Bm"], td["Cm"], pd, h, c)
        if t % 16 == 0 or t == w.decode_steps - 1:
            torch.cuda.synchronize()
            yc, hc, cc = f64(y), None, None
        for (b, ch) in pairs:
            hs, cs = st[(b, ch)]
            one = {k: v[b:b + 1, ch:ch + 1] if k in ("x", "dt", "z") else v[b:b + 1] for k, v in tok.items()}
            ps = {k: v[ch:ch + 1] for k, v in prm.items()}
            yr, hs, cs = oracle.decode_step(one, ps, hs, cs)
            st[(b, ch)] = (hs, cs)
            if t % 16 == 0 or t == w.decode_steps - 1:
                assert_close(yc[b, ch], yr[0, 0], TAU[w.io], f"{name} decode y step {t} [{b},{ch}]")
    torch.cuda.synchronize()
    for (b, ch) in pairs:
        hs, cs = st[(b, ch)]
        assert_close(h[b, ch], hs[0, 0], TAU[w.io], f"{name} decode h [{b},{ch}]")
        assert_bitwise(c[b, ch], cs[0, 0], f"{name} decode conv [{b},{ch}]")


@pytest.mark.timeout(300)
def test_slice7b_prefill_and_decode():
    w, prm, pd, s, (y, h, c), pairs, ref = prefill_and_check("slice7b")
    decode_and_check("slice7b", w, prm, pd, h, c, pairs, ref)


@pytest.mark.timeout(300)
def test_mamba2_8b_prefill_and_decode():
    w, prm, pd, s, (y, h, c), pairs, ref = prefill_and_check("mamba2.8b", k=16)
    del s, y
    torch.cuda.empty_cache()
    decode_and_check("mamba2.8b", w, prm, pd, h, c, pairs, ref)


@pytest.mark.timeout(300)
def test_long64k_prefill():
    prefill_and_check("long64k", k=16)
