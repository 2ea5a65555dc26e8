"""HIP path vs the fp64 oracle on the same seeded inputs (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_causal_amd as ssm
from selective_state_space_causal_amd import inputs as I
from tests import parity_cases as PC
from tests.gpu_common import DEV, TAU, assert_bitwise, assert_close, dev, f64, note, sample_pairs, threads

pytestmark = pytest.mark.gpu


def run(seq, prm, gate=True, **kw):
    s = dev(seq)
    return ssm.prefill(s["x"], s["dt"], s["z"] if gate else None, s["Bm"], s["Cm"], dev(prm), **kw)


def check_full(seq, prm, io, gate=True, what="", **kw):
    y, h, c = run(seq, prm, gate, **kw)
    torch.cuda.synchronize()
    yr, hr, cr = oracle.prefill(seq, prm, nthreads=threads(), gate=gate)
    ey = assert_close(y, yr, TAU[io], f"{what} y")
    eh = assert_close(h, hr, TAU[io], f"{what} h")
    assert_bitwise(c, cr, f"{what} conv")
    return ey, eh


def test_tiny_fp32_workload():
    w = I.WORKLOADS["tiny"]
    note(f"tiny: B={w.batch} L={w.seqlen} D={w.d_inner} N={w.d_state} {w.io}")
    prm = I.make_params(w.d_inner, w.d_state)
    seq = I.make_sequence(w.batch, w.seqlen, w.d_inner, w.d_state, w.io)
    ey, eh = check_full(seq, prm, w.io, what="tiny")
    note(f"tiny max err y {ey:.2e} h {eh:.2e}")


@pytest.mark.parametrize("params", ["workload", "distinct"])
def test_mamba130m_workload_full_tensors(params):
    """The workload's own parameter distributions, and per-channel ones (make_params_distinct)
    on the same inputs; it runs the 12-channel workgroup shape, with a ragged last group."""
    w = I.WORKLOADS["mamba130m"]
    note(f"mamba130m ({params} params): B={w.batch} L={w.seqlen} D={w.d_inner} N={w.d_state} {w.io}")
    mk = I.make_params if params == "workload" else I.make_params_distinct
    prm = mk(w.d_inner, w.d_state)
    seq = I.make_sequence(w.batch, w.seqlen, w.d_inner, w.d_state, w.io)
    ey, eh = check_full(seq, prm, w.io, what="mamba130m")
    note(f"mamba130m max err y {ey:.2e} h {eh:.2e}")


@pytest.mark.parametrize("B,L,D,N,io,gate,cb", PC.EDGE)
def test_edge_shapes(B, L, D, N, io, gate, cb):
    note(f"edge B={B} L={L} D={D} N={N} {io} gate={gate} conv_b={cb}")
    prm, seq = PC.edge_inputs(B, L, D, N, io, gate, cb)
    check_full(seq, prm, io, gate, what=f"edge{B},{L},{D},{N}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_chunked_prefill_from_cache(io):
    """prefill(L1) then prefill(L2) resumed from its cache == prefill(L1 + L2)."""
    B, D, N, L1, L2 = 2, 70, 16, 300, 211
    note(f"chunked prefill {io}")
    prm = I.make_params_distinct(D, N, seed=3)
    seq = I.make_sequence(B, L1 + L2, D, N, io, seed=3)
    part = lambda s, a, b: {k: (v[:, :, a:b] if k in ("x", "dt", "z") else v[:, a:b]).contiguous()
                            for k, v in s.items()}
    y1, h1, c1 = run(part(seq, 0, L1), prm)
    s2 = dev(part(seq, L1, L1 + L2))
    y2, h2, c2 = ssm.prefill(s2["x"], s2["dt"], s2["z"], s2["Bm"], s2["Cm"], dev(prm), h0=h1, conv0=c1)
    torch.cuda.synchronize()
    yr, hr, cr = oracle.prefill(seq, prm, nthreads=threads())
    assert_close(torch.cat([y1, y2], 2), yr, TAU[io], "chunked y")
    assert_close(h2, hr, TAU[io], "chunked h")
    assert_bitwise(c2, cr, "chunked conv")


@pytest.mark.parametrize("io,B,D,N", PC.DECODE)
def test_decode_steps_match_oracle(io, B, D, N):
    """Prefill, then T single-token steps from the cache; y, h each step, conv bitwise each step."""
    note(f"decode {io} B={B} D={D} N={N}")
    prm, seq, toks = PC.decode_inputs(io, B, D, N)
    _, h, c = run(seq, prm)
    _, hr, cr = oracle.prefill(seq, prm)
    pd = dev(prm)
    for t, tok in enumerate(toks):
        td = dev(tok)
        y = ssm.decode_step(td["x"], td["dt"], td["z"], td["Bm"], td["Cm"], pd, h, c)
        yr, hr, cr = oracle.decode_step(tok, prm, hr, cr)
        assert_close(y, yr, TAU[io], f"decode y step {t}")
        assert_close(h, hr, TAU[io], f"decode h step {t}")
        assert_bitwise(c, cr, f"decode conv step {t}")


def test_decode_equals_longer_prefill():
    """State caching invariant on the GPU: prefill(L1) + L2 decode steps == prefill(L1 + L2)."""
    B, D, N, L1, L2 = 2, 96, 16, 200, 40
    prm = I.make_params_distinct(D, N, seed=9)
    seq = I.make_sequence(B, L1 + L2, D, N, "bf16", seed=9)
    yf, hf, cf = run(seq, prm)
    s = dev(seq)
    _, h, c = ssm.prefill(s["x"][:, :, :L1].contiguous(), s["dt"][:, :, :L1].contiguous(),
                          s["z"][:, :, :L1].contiguous(), s["Bm"][:, :L1].contiguous(),
                          s["Cm"][:, :L1].contiguous(), dev(prm))
    pd = dev(prm)
    for t in range(L1, L1 + L2):
        y = ssm.decode_step(s["x"][:, :, t].contiguous(), s["dt"][:, :, t].contiguous(), s["z"][:, :, t].contiguous(),
                            s["Bm"][:, t].contiguous(), s["Cm"][:, t].contiguous(), pd, h, c)
        assert_close(y, f64(yf[:, :, t]), TAU["bf16"], f"step {t} vs prefill")
    assert_close(h, f64(hf), 1e-4, "h after decode vs prefill")
    assert_bitwise(c, f64(cf), "conv after decode vs prefill")


def test_channel_and_batch_slices_are_bitwise():
    """Channel locality on the GPU: a channel slice (or batch row) run alone reproduces the
    full run bit for bit when the decomposition is pinned with chunk_hint."""
    B, L, D, N = 3, 300, 200, 16
    prm = I.make_params_distinct(D, N, seed=11)
    seq = I.make_sequence(B, L, D, N, "bf16", seed=11)
    y, h, c = run(seq, prm, chunk_hint=1)
    for lo, hi in ((0, 64), (64, 65), (65, 200)):
        ps = {k: v[lo:hi].contiguous() for k, v in prm.items()}
        ss = {k: (v[:, lo:hi].contiguous() if k in ("x", "dt", "z") else v) for k, v in seq.items()}
        ys, hs, cs = run(ss, ps, chunk_hint=1)
        assert torch.equal(ys.view(torch.int16), y[:, lo:hi].view(torch.int16))
        assert torch.equal(hs, h[:, lo:hi]) and torch.equal(cs, c[:, lo:hi])
    for b in range(B):
        sb = {k: v[b:b + 1].contiguous() for k, v in seq.items()}
        yb, hb, _ = run(sb, prm, chunk_hint=1)
        assert torch.equal(yb.view(torch.int16), y[b:b + 1].view(torch.int16)) and torch.equal(hb, h[b:b + 1])


def test_pow2_scaling_bitwise():
    """Dskip = 0: doubling C doubles y; doubling B doubles h and y (exact in binary fp).  The
    workload's parameters keep every decay well above the fp32 subnormal range, where a doubled
    product could escape a flush to zero that the plain one takes."""
    B, L, D, N = 2, 150, 70, 16
    prm = I.make_params(D, N, seed=13)
    prm["Dskip"] = torch.zeros_like(prm["Dskip"])
    seq = I.make_sequence(B, L, D, N, "f32", seed=13)
    y, h, _ = run(seq, prm)
    y2, h2, _ = run(dict(seq, Cm=seq["Cm"] * 2), prm)
    assert torch.equal(y2, 2 * y) and torch.equal(h2, h)
    y3, h3, _ = run(dict(seq, Bm=seq["Bm"] * 2), prm)
    assert torch.equal(h3, 2 * h) and torch.equal(y3, 2 * y)


def test_deterministic_and_in_bounds():
    """Two runs are bitwise equal, and nothing is written outside the outputs (canaries)."""
    B, L, D, N = 2, 333, 97, 16
    prm = dev(I.make_params_distinct(D, N, seed=17))
    s = dev(I.make_sequence(B, L, D, N, "bf16", seed=17))
    pad = 4096
    outs = []
    for _ in range(2):
        ybuf = torch.full((B * D * L + 2 * pad,), 12345.0, dtype=torch.bfloat16, device=DEV)
        hbuf = torch.full((B * D * N + 2 * pad,), -7.0, device=DEV)
        cbuf = torch.full((B * D * 3 + 2 * pad,), -9.0, device=DEV)
        y = ybuf[pad:pad + B * D * L].view(B, D, L)
        h = hbuf[pad:pad + B * D * N].view(B, D, N)
        c = cbuf[pad:pad + B * D * 3].view(B, D, 3)
        ssm.prefill(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], prm, y=y, h_out=h, conv_out=c)
        torch.cuda.synchronize()
        for buf, val in ((ybuf, 12345.0), (hbuf, -7.0), (cbuf, -9.0)):
            assert torch.all(buf[:pad] == val) and torch.all(buf[-pad:] == val), "write outside an output"
        outs.append((y.clone(), h.clone(), c.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_cache_roundtrip_through_host():
    """Copying the cache to the host and back, then resuming, equals resuming directly."""
    B, L, D, N = 1, 100, 64, 16
    prm = dev(I.make_params_distinct(D, N, seed=19))
    s = dev(I.make_sequence(B, L, D, N, "bf16", seed=19))
    _, h, c = ssm.prefill(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], prm)
    h2, c2 = h.cpu().to(DEV), c.cpu().to(DEV)
    tok = dev(I.make_decode_token(B, D, N, 0, "bf16", seed=19))
    ya = ssm.decode_step(tok["x"], tok["dt"], tok["z"], tok["Bm"], tok["Cm"], prm, h, c)
    yb = ssm.decode_step(tok["x"], tok["dt"], tok["z"], tok["Bm"], tok["Cm"], prm, h2, c2)
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)) and torch.equal(h, h2) and torch.equal(c, c2)


def test_error_paths_with_real_tensors():
    B, L, D, N = 1, 64, 32, 16
    prm = dev(I.make_params(D, N))
    s = dev(I.make_sequence(B, L, D, N, "bf16"))
    with pytest.raises(ssm.SsmError) as e:       # y aliases x
        ssm.prefill(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], prm, y=s["x"])
    assert e.value.status == 5
    big = torch.empty(B * D * L + 8, dtype=torch.bfloat16, device=DEV)
    x_mis = big[1:1 + B * D * L].view(B, D, L)   # 2-byte offset: misaligned
    x_mis.copy_(s["x"])
    with pytest.raises(ssm.SsmError) as e:
        ssm.prefill(x_mis, s["dt"], s["z"], s["Bm"], s["Cm"], prm)
    assert e.value.status == 4
    # given outputs of the wrong size are refused by the binding before any launch
    with pytest.raises(ValueError):
        ssm.prefill(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], prm, y=torch.empty(B, D, L - 8, dtype=torch.bfloat16,
                                                                                   device=DEV))
    with pytest.raises(ValueError):
        ssm.prefill(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], prm, h_out=torch.empty(B, D, N - 1, device=DEV))
    with pytest.raises(TypeError):
        ssm.prefill(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], prm, conv_out=torch.empty(B, D, 3, device=DEV,
                                                                                          dtype=torch.float64))
    tok = dev(I.make_decode_token(B, D, N, 0, "bf16"))
    h, c = torch.zeros(B, D, N, device=DEV), torch.zeros(B, D, 3, device=DEV)
    with pytest.raises(ValueError):
        ssm.decode_step(tok["x"], tok["dt"], tok["z"], tok["Bm"], tok["Cm"], prm, h, c,
                        y_t=torch.empty(B, D // 2, dtype=torch.bfloat16, device=DEV))


@pytest.mark.parametrize("B,L,D,io", PC.WINDOWED)
def test_windowed_kernel_shapes(B, L, D, io):
    """The windowed (lanes over time) prefill, forced with chunk_hint=8, against the oracle:
    fresh, then without a gate resumed from a random cache."""
    note(f"windowed B={B} L={L} D={D} {io}")
    prm, seq = PC.windowed_inputs(B, L, D, io)
    check_full(seq, prm, io, what=f"windowed{B},{L},{D}", chunk_hint=8)
    s = dev(seq)
    h0, c0 = PC.random_cache(B, D, 16, seed=L, io=io)
    y, h, c = ssm.prefill(s["x"], s["dt"], None, s["Bm"], s["Cm"], dev(prm), h0=h0.to(DEV), conv0=c0.to(DEV),
                          chunk_hint=8)
    yr, hr, cr = oracle.scan(seq["x"], seq["dt"], None, seq["Bm"], seq["Cm"], prm["A"], prm["Dskip"],
                             prm["dt_bias"], prm["conv_w"], prm["conv_b"], h0=f64(h0), conv0=f64(c0))
    assert_close(y, yr, TAU[io], "windowed resumed y")
    assert_close(h, hr, TAU[io], "windowed resumed h")
    assert_bitwise(c, cr, "windowed resumed conv")


def test_windowed_and_sequential_agree():
    B, L, D, N = 2, 3000, 40, 16
    prm = I.make_params_distinct(D, N, seed=21)
    seq = I.make_sequence(B, L, D, N, "f32", seed=21)
    ya, ha, ca = run(seq, prm, chunk_hint=8)
    yb, hb, cb = run(seq, prm, chunk_hint=1)
    assert_close(ya, f64(yb), 1e-4, "windowed vs sequential y")
    assert_close(ha, f64(hb), 1e-4, "windowed vs sequential h")
    assert torch.equal(ca, cb)


@pytest.mark.parametrize("L,D", [(1024, 24), (777, 9)])
def test_bf16_output_is_rne_of_fp32_output(L, D):
    """Same bf16-representable inputs through the fp32-io and bf16-io paths: the arithmetic is
    identical, so the bf16 outputs must be the round-to-nearest-even of the fp32 outputs (bit for
    bit) and the fp32 state identical -- for prefill and for a decode step."""
    B, N = 2, 16
    prm = dev(I.make_params_distinct(D, N, seed=41))
    s16 = dev(I.make_sequence(B, L, D, N, "bf16", seed=41))
    s32 = {k: v.float() for k, v in s16.items()}
    y16, h16, c16 = ssm.prefill(s16["x"], s16["dt"], s16["z"], s16["Bm"], s16["Cm"], prm)
    y32, h32, c32 = ssm.prefill(s32["x"], s32["dt"], s32["z"], s32["Bm"], s32["Cm"], prm)
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(h16, h32) and torch.equal(c16, c32)
    t16 = dev(I.make_decode_token(B, D, N, 0, "bf16", seed=41))
    t32 = {k: v.float() for k, v in t16.items()}
    u16 = ssm.decode_step(t16["x"], t16["dt"], t16["z"], t16["Bm"], t16["Cm"], prm, h16, c16)
    u32 = ssm.decode_step(t32["x"], t32["dt"], t32["z"], t32["Bm"], t32["Cm"], prm, h32, c32)
    assert torch.equal(u16.view(torch.int16), u32.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(h16, h32) and torch.equal(c16, c32)


def test_launch_shapes_agree_bitwise():
    """The bf16 prefill picks its workgroup shape (8, 12 or 16 channels, in state groups of 8,
    4 or 2) from the number of workgroup rounds the launch needs, so the same channel runs in
    different shapes depending on what else is in the launch.  Per channel the arithmetic is
    the same, so every run must give the same bits (the channel-slice invariant, across launch
    shapes).  On a 256-CU MI355X: all 4 rows of 3990 channels and one row alone run 16 channels
    per workgroup; a 2990-channel slice runs 12; a 1995-channel slice runs 8 (each with a
    ragged last workgroup).  With per-channel parameters, the channels at the edges of the
    workgroups, the ragged last group of each shape among them, are also checked against the
    oracle."""
    B, L, D, N = 4, 1040, 3990, 16
    note(f"launch shapes: B={B} L={L} D={D}")
    prm_h = I.make_params_distinct(D, N, seed=51)
    prm = dev(prm_h)
    seq = I.make_sequence_device(B, L, D, N, "bf16", seed=51, device=DEV)
    y, h, c = ssm.prefill(seq["x"], seq["dt"], seq["z"], seq["Bm"], seq["Cm"], prm)
    for b in range(B):
        for n in (D, 2990, 1995):
            one = {k: (v[b:b + 1, :n] if k in ("x", "dt", "z") else v[b:b + 1]).contiguous() for k, v in seq.items()}
            pn = {k: (None if v is None else v[:n].contiguous()) for k, v in prm.items()}
            yb, hb, cb = ssm.prefill(one["x"], one["dt"], one["z"], one["Bm"], one["Cm"], pn)
            torch.cuda.synchronize()
            assert torch.equal(yb[0].view(torch.int16), y[b, :n].view(torch.int16)), (b, n)
            assert torch.equal(hb[0], h[b, :n]) and torch.equal(cb[0], c[b, :n]), (b, n)
    edges = {0, 1, 7, 8, 11, 12, 15, 16, 1991, 1992, 1993, 1994, 2987, 2988, 2989, 3983, 3984, 3989}
    rnd = np.random.default_rng(51).integers(0, D, 8)
    pairs = [(b, int(ch)) for b in (0, B - 1) for ch in sorted(edges | set(rnd.tolist()))]
    for (b, ch), (yr, hr, cr) in zip(pairs, oracle.scan_channels(seq, prm_h, pairs)):
        assert_close(y[b, ch], yr, TAU["bf16"], f"shapes y[{b},{ch}]")
        assert_close(h[b, ch], hr, TAU["bf16"], f"shapes h[{b},{ch}]")
        assert_bitwise(c[b, ch], cr, f"shapes conv[{b},{ch}]")


# The method's degenerate regimes (tests/parity_cases.py), each against the oracle through both
# prefill decompositions and a few decode steps.
@pytest.mark.parametrize("chunk_hint", [0, 1])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("regime", PC.REGIMES)
def test_degenerate_regimes(regime, io, chunk_hint):
    B, L, D, N, T = 2, 600, 24, 16, 3  # L: one full 512-token window and a ragged one
    note(f"regime {regime} {io} chunk_hint={chunk_hint}")
    prm, seq = PC.regime(regime, PC.regime_params(D, N), I.make_sequence(B, L, D, N, io, seed=17))
    y, h, c = run(seq, prm, chunk_hint=chunk_hint)
    torch.cuda.synchronize()
    yr, hr, cr = oracle.prefill(seq, prm, nthreads=threads())
    assert_close(y, yr, TAU[io], f"{regime} y")
    assert_close(h, hr, TAU[io], f"{regime} h")
    assert_bitwise(c, cr, f"{regime} conv")
    pd = dev(prm)
    for t in range(T):
        _, tok = PC.regime(regime, prm, I.make_decode_token(B, D, N, t, io, seed=17))
        td = dev(tok)
        yt = ssm.decode_step(td["x"], td["dt"], td["z"], td["Bm"], td["Cm"], pd, h, c)
        yrt, hr, cr = oracle.decode_step(tok, prm, hr, cr)
        assert_close(yt, yrt, TAU[io], f"{regime} decode y step {t}")
        assert_close(h, hr, TAU[io], f"{regime} decode h step {t}")
        assert_bitwise(c, cr, f"{regime} decode conv step {t}")
