"""Full-size workloads on the GPU, checked against the oracle on sampled channels (the
recurrence is channel-local, so each sampled (b, c) is computed exactly and alone).

Each workload runs with its own parameter distributions and with per-channel ones
(make_params_distinct) on the same inputs, in the launch shape the benchmark times.  Decode
steps are checked at every step: y, the state h and the conv window of every sampled channel."""
import pytest
import torch

import oracle
import selective_state_space_causal_amd as ssm
from selective_state_space_causal_amd import inputs as I
from tests.gpu_common import DEV, TAU, assert_bitwise, assert_close, dev, f64, note, sample_pairs

pytestmark = pytest.mark.gpu


def params(w, kind):
    if kind == "workload":
        return I.make_params(w.d_inner, w.d_state, dt_range=w.dt_range)
    return I.make_params_distinct(w.d_inner, w.d_state)


def prefill_and_check(name, kind, s=None, k=24):
    w = I.WORKLOADS[name]
    if s is None:
        note(f"{name}: B={w.batch} L={w.seqlen} D={w.d_inner} N={w.d_state} {w.io}: generating")
        s = I.make_sequence_device(w.batch, w.seqlen, w.d_inner, w.d_state, w.io, device=DEV)
    prm = params(w, kind)
    pd = dev(prm)
    note(f"{name} ({kind} params): prefill")
    y, h, c = ssm.prefill(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], pd)
    torch.cuda.synchronize()
    pairs = sample_pairs(w.batch, w.d_inner, k)
    note(f"{name} ({kind} params): oracle on {len(pairs)} channels")
    ref = oracle.scan_channels(s, prm, pairs)
    for (b, ch), (yr, hr, cr) in zip(pairs, ref):
        assert_close(y[b, ch], yr, TAU[w.io], f"{name} y[{b},{ch}]")
        assert_close(h[b, ch], hr, TAU[w.io], f"{name} h[{b},{ch}]")
        assert_bitwise(c[b, ch], cr, f"{name} conv[{b},{ch}]")
    return w, prm, pd, s, (y, h, c), pairs, ref


def decode_and_check(name, w, prm, pd, h, c, pairs, ref):
    """The workload's decode steps from the prefill's cache; at every step the sampled
    channels' y, h and conv window against the oracle stepping those channels alone."""
    st = {p: (r[1][None, None], r[2][None, None]) for p, r in zip(pairs, ref)}
    bi = torch.tensor([b for b, _ in pairs], device=DEV)
    ci = torch.tensor([ch for _, ch in pairs], device=DEV)
    tau = TAU[w.io]
    note(f"{name}: {w.decode_steps} decode steps, every one checked")
    for t in range(w.decode_steps):
        tok = I.make_decode_token(w.batch, w.d_inner, w.d_state, t, w.io)
        td = dev(tok)
        y = ssm.decode_step(td["x"], td["dt"], td["z"], td["Bm"], td["Cm"], pd, h, c)
        yc, hc, cc = f64(y[bi, ci]), f64(h[bi, ci]), f64(c[bi, ci])
        for i, (b, ch) in enumerate(pairs):
            hs, cs = st[(b, ch)]
            one = {k: v[b:b + 1, ch:ch + 1] if k in ("x", "dt", "z") else v[b:b + 1] for k, v in tok.items()}
            ps = {k: v[ch:ch + 1] for k, v in prm.items()}
            yr, hs, cs = oracle.decode_step(one, ps, hs, cs)
            st[(b, ch)] = (hs, cs)
            assert_close(yc[i], yr[0, 0], tau, f"{name} decode y step {t} [{b},{ch}]", step=t)
            assert_close(hc[i], hs[0, 0], tau, f"{name} decode h step {t} [{b},{ch}]", step=t)
            assert_bitwise(cc[i], cs[0, 0], f"{name} decode conv step {t} [{b},{ch}]")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind", ["workload", "distinct"])
def test_slice7b_prefill_and_decode(kind):
    w, prm, pd, s, (y, h, c), pairs, ref = prefill_and_check("slice7b", kind)
    decode_and_check("slice7b", w, prm, pd, h, c, pairs, ref)


@pytest.mark.timeout(600)
def test_mamba2_8b_prefill_and_decode():
    s = None
    for kind in ("workload", "distinct"):
        w, prm, pd, s, (y, h, c), pairs, ref = prefill_and_check("mamba2.8b", kind, s=s, k=16)
        del y
        torch.cuda.empty_cache()
        decode_and_check("mamba2.8b", w, prm, pd, h, c, pairs, ref)
        del h, c


@pytest.mark.timeout(300)
def test_long64k_prefill():
    s = None
    for kind in ("workload", "distinct"):
        *_, s, _, _, _ = prefill_and_check("long64k", kind, s=s, k=16)
