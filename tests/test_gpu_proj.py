"""Channel-sliced projections, the conv front and one rank's mixer layer on the GPU against the
fp64 oracle (oracle/proj.py, and the scan's C oracle for the layer).

Projections: the GPU accumulates in fp32 (hipBLASLt, order unknown), so each output is held
to |gpu - ref| <= K * 2^-24 * sum_k |W_mk in_k| (the worst case of any fp32 summation order)
plus, for bf16 output, the final round to nearest even (at most 2^-8 of the value).  The conv
front: fp32 arithmetic then the io rounding.  The layer: the oracle rounds every intermediate
tensor to the io dtype at the same points as the GPU, and the output is held to the scan's
tolerance, 2e-2 (1 + |ref|) for bf16 io."""
import numpy as np
import pytest
import torch

import oracle
from oracle import proj as P
from selective_state_space_causal_amd import _lib as L
from selective_state_space_causal_amd import inputs as I
from selective_state_space_causal_amd import layer
from tests.gpu_common import DEV, note, threads

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
DT = {"bf16": torch.bfloat16, "f32": torch.float32}
REF = {L.PROJ_IN: P.in_proj, L.PROJ_DT: P.dt_proj, L.PROJ_X: P.x_proj, L.PROJ_OUT: P.out_proj}
NAMES = {L.PROJ_IN: "in", L.PROJ_X: "x", L.PROJ_DT: "dt", L.PROJ_OUT: "out"}


@pytest.fixture(scope="module")
def pj():
    p = L.Projector(DEV)
    yield p
    p.close()


def bound(kind, x, w, ref, out_bf16):
    K = w.shape[1]
    mag = REF[kind](np.abs(x.double().numpy()), np.abs(w.double().numpy()))
    b = K * U * mag
    if out_bf16:
        b = b + 2.0 ** -8 * (np.abs(ref) + b)
    return b


@pytest.mark.parametrize("kind", [L.PROJ_IN, L.PROJ_X, L.PROJ_DT, L.PROJ_OUT])
@pytest.mark.parametrize("io,od", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")])
@pytest.mark.parametrize("B,Ls,K,M", [(2, 64, 32, 48), (1, 33, 17, 5), (3, 7, 3, 9), (2, 520, 96, 40),
                                      # one token per row: the streaming matrix-vector kernel (batch
                                      # groups of 8, 4, 2, 1; ragged rows per wave and pieces per lane)
                                      (1, 1, 4096, 64), (3, 1, 96, 40), (8, 1, 2048, 24), (11, 1, 64, 33),
                                      (16, 1, 520, 17), (2, 1, 20, 7),
                                      # ... and the GEMM when it does not apply (K not a whole
                                      # number of 16-byte pieces, more than 16 rows)
                                      (1, 1, 17, 5), (20, 1, 64, 16),
                                      # token-major in, channel-major out, K a multiple of 16 up to
                                      # 256: the small-K kernel (tiles across batch rows, channel
                                      # groups of 512 with a ragged last one, K 16 and 256)
                                      (3, 200, 256, 600), (1, 40, 16, 1), (2, 24, 160, 130)])
def test_projection_matches_oracle(pj, kind, io, od, B, Ls, K, M):
    note(f"proj {NAMES[kind]} io={io} out={od} B={B} L={Ls} K={K} M={M}")
    g = torch.Generator().manual_seed(B * 1000 + Ls * 10 + K + kind)
    tm = kind in (L.PROJ_IN, L.PROJ_DT)
    x = torch.randn((B, Ls, K) if tm else (B, K, Ls), generator=g).to(DT[io])
    w = (torch.randn(M, K, generator=g) / K ** 0.5).to(DT[io])
    out = pj(kind, x.to(DEV), w.to(DEV), out_dtype=DT[od])
    torch.cuda.synchronize()
    assert tuple(out.shape) == ((B, M, Ls) if tm else (B, Ls, M))
    ref = REF[kind](x, w)
    got = out.double().cpu().numpy()
    b = bound(kind, x, w, ref, od == "bf16")
    err = np.abs(got - ref)
    i = np.unravel_index(int(np.argmax(err - b)), err.shape)
    assert np.all(err <= b), f"{i}: gpu {got[i]!r} ref {ref[i]!r} bound {b[i]:.3e}"


def test_projection_errors(pj):
    x = torch.randn(1, 64, 32, device=DEV, dtype=torch.bfloat16)
    w = torch.randn(16, 32, device=DEV, dtype=torch.bfloat16)
    buf = torch.empty(16 * 64 + 8, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(L.SsmError) as e:
        pj(L.PROJ_IN, x, w, out=buf[1:1 + 16 * 64].view(1, 16, 64))   # 2-byte offset: not 16-byte aligned
    assert e.value.status == 4
    with pytest.raises(ValueError):
        pj(L.PROJ_IN, x, torch.randn(16, 31, device=DEV, dtype=torch.bfloat16))


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("B,D,Ls", [(2, 8, 64), (1, 5, 37), (2, 3, 1), (3, 16, 200), (1, 4, 12)])
@pytest.mark.parametrize("resume", [False, True])
def test_conv_silu_matches_oracle(io, B, D, Ls, resume):
    note(f"conv_silu io={io} B={B} D={D} L={Ls} resume={resume}")
    prm = I.make_params_distinct(D, 16)
    g = torch.Generator().manual_seed(B * 100 + D * 10 + Ls)
    x = torch.randn(B, D, Ls, generator=g).to(DT[io])
    conv0 = torch.randn(B, D, 3, generator=g).to(DT[io]).float() if resume else None
    pd = {k: v.to(DEV) for k, v in prm.items() if v is not None}
    u = L.conv_silu(x.to(DEV), pd, None if conv0 is None else conv0.to(DEV))
    torch.cuda.synchronize()
    ref = P.conv_silu(x, prm["conv_w"], prm.get("conv_b"), None if conv0 is None else conv0.double().numpy())
    got = u.double().cpu().numpy()
    tol = 2.0 ** -8 * np.abs(ref) + 1e-6 * (1 + np.abs(ref)) if io == "bf16" else 2e-6 * (1 + np.abs(ref))
    assert np.all(np.abs(got - ref) <= tol), float(np.max(np.abs(got - ref) - tol))


def test_conv_silu_resume_is_bitwise():
    """Running tokens [L1, L) with the last three raw inputs before L1 as history reproduces
    the tail of the full run bit for bit (the arithmetic per token is the same)."""
    prm = {k: v.to(DEV) for k, v in I.make_params_distinct(12, 16).items() if v is not None}
    x = torch.randn(2, 12, 96, device=DEV).to(torch.bfloat16)
    full = L.conv_silu(x, prm)
    for L1 in (8, 40, 88):
        hist = x[:, :, L1 - 3:L1].float().contiguous()
        tail = L.conv_silu(x[:, :, L1:].contiguous(), prm, hist)
        torch.cuda.synchronize()
        assert torch.equal(tail, full[:, :, L1:]), L1


@pytest.mark.parametrize("rows,out_f32,fused", [(2, False, True), (1, False, True), (2, True, True),
                                                (2, False, False)])
def test_layer_small_matches_oracle(pj, rows, out_f32, fused):
    """Two batch rows run in_proj as two GEMMs (x rows, z rows); one row runs it as one GEMM
    over the stacked weight.  The conv front and x_proj fused (the stacked x_proj weight) or
    as conv_silu then three GEMMs.  The out partial in bf16 (default) or fp32."""
    w8 = I.LAYERS["layer_small"]
    note(f"layer {w8} rows={rows} out_f32={out_f32}")
    prm = I.make_params_distinct(w8.d_inner, w8.d_state)
    wts = I.make_proj_weights(w8.d_model, w8.d_inner, w8.dt_rank, w8.d_state, w8.io)
    hidden = I.make_hidden(w8.batch, w8.seqlen, w8.d_model, w8.io)[:rows].contiguous()
    wd = {k: v.to(DEV) for k, v in wts.items() if k not in ("in_x", "in_z")}
    wd["in_x"], wd["in_z"] = wd["in_xz"][:w8.d_inner], wd["in_xz"][w8.d_inner:]
    if not fused:
        del wd["x_all"]
    hd = hidden.to(DEV)
    assert layer._stacked_in_proj(hd, wd) == (rows == 1)
    assert layer._fused_conv_xproj(hd, wd) == fused
    out, h, c = layer.mixer_prefill(hd, wd, {k: v.to(DEV) for k, v in prm.items() if v is not None}, pj,
                                    out_dtype=torch.float32 if out_f32 else None)
    torch.cuda.synchronize()
    assert out.dtype == (torch.float32 if out_f32 else hidden.dtype)
    ref, h_ref, c_ref = P.layer_prefill(hidden, wts, prm, w8.io, nthreads=threads(), out_io=not out_f32)
    got = out.double().cpu().numpy()
    err = np.abs(got - ref) / (1 + np.abs(ref))
    note(f"layer: max err {err.max():.3e}")
    assert err.max() <= 2e-2
    herr = np.abs(h.double().cpu().numpy() - h_ref) / (1 + np.abs(h_ref))
    assert herr.max() <= 2e-2


def test_in_proj_full_size_sampled(pj):
    """in_proj of the 7B-class layer at its real size ([1, 32768, 4096] x [2048, 4096], bf16):
    sampled outputs against fp64 dot products."""
    w8 = I.LAYERS["layer7b"]
    hidden = I.make_hidden(w8.batch, w8.seqlen, w8.d_model, w8.io, device=DEV)
    wx = I.make_proj_weights(w8.d_model, w8.d_inner, w8.dt_rank, w8.d_state, w8.io, device=DEV)["in_x"]
    x = pj(L.PROJ_IN, hidden, wx)
    torch.cuda.synchronize()
    g = np.random.default_rng(0)
    cs = g.integers(0, w8.d_inner, 400)
    ts = g.integers(0, w8.seqlen, 400)
    hs = hidden[0, torch.tensor(ts, device=DEV)].double().cpu().numpy()   # [400, d_model]
    ws = wx[torch.tensor(cs, device=DEV)].double().cpu().numpy()
    ref = np.sum(hs * ws, axis=1)
    mag = np.sum(np.abs(hs * ws), axis=1)
    got = x[0, torch.tensor(cs, device=DEV), torch.tensor(ts, device=DEV)].double().cpu().numpy()
    b = w8.d_model * U * mag
    b = b + 2.0 ** -8 * (np.abs(ref) + b)
    assert np.all(np.abs(got - ref) <= b)


def test_dt_proj_full_size_sampled(pj):
    """dt_proj of the 7B-class layer at its real size ([1, 32768, 256] x [2048, 256], bf16, the
    small-K kernel): sampled outputs against fp64 dot products, and the first and last tiles whole."""
    w8 = I.LAYERS["layer7b"]
    D, Ls, R = w8.d_inner, w8.seqlen, w8.dt_rank
    g = torch.Generator(device=DEV).manual_seed(3)
    lr = torch.randn(1, Ls, R, generator=g, device=DEV).to(torch.bfloat16)
    wdt = I.make_proj_weights(w8.d_model, D, R, w8.d_state, w8.io, device=DEV)["dt"]
    dt = pj(L.PROJ_DT, lr, wdt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    cs = np.concatenate([rng.integers(0, D, 600), np.arange(D), np.arange(D)])
    ts = np.concatenate([rng.integers(0, Ls, 600), np.zeros(D, dtype=np.int64), np.full(D, Ls - 1)])
    ls = lr[0, torch.tensor(ts, device=DEV)].double().cpu().numpy()
    ws = wdt[torch.tensor(cs, device=DEV)].double().cpu().numpy()
    ref = np.sum(ls * ws, axis=1)
    mag = np.sum(np.abs(ls * ws), axis=1)
    got = dt[0, torch.tensor(cs, device=DEV), torch.tensor(ts, device=DEV)].double().cpu().numpy()
    b = R * U * mag
    b = b + 2.0 ** -8 * (np.abs(ref) + b)
    assert np.all(np.abs(got - ref) <= b)


def conv_magnitude(x, conv_w, conv_b, conv0):
    """|conv_b| + sum_k |conv_w[k]| |xi[t - 3 + k]|: the scale of the conv sum's fp32 rounding."""
    xa = np.abs(x.double().numpy())
    B, D, Ls = xa.shape
    hist = np.zeros((B, D, 3)) if conv0 is None else np.abs(conv0)
    xi = np.concatenate([hist, xa], axis=2)
    wa = np.abs(conv_w.double().numpy())
    m = np.zeros((B, D, Ls)) if conv_b is None else \
        np.broadcast_to(np.abs(conv_b.double().numpy())[None, :, None], (B, D, Ls)).copy()
    for k in range(4):
        m += wa[None, :, k, None] * xi[:, :, k:k + Ls]
    return m


def bf16_flip_ulps(u64, scale):
    """For fp64 values u64 that the GPU computes in fp32 (error within 2^-18 |u| + 2^-20 scale)
    and then rounds to bf16: the bf16 ulp where that rounding could go either way (the value is
    that close to a midpoint between two bf16 numbers), else 0."""
    a = np.abs(u64)
    nz = a > 1e-30
    e = np.floor(np.log2(np.where(nz, a, 1.0)))
    ulp = np.exp2(e - 7)
    f = a / ulp
    dist = np.abs(f - np.floor(f) - 0.5) * ulp
    delta = 2.0 ** -18 * a + 2.0 ** -20 * scale
    return np.where(nz & (dist <= delta), ulp, 0.0)


@pytest.mark.parametrize("B,Ls,D,R,N,resume", [(1, 256, 64, 8, 16, False), (2, 200, 96, 256, 16, True),
                                                (1, 136, 40, 300, 16, False), (3, 64, 2048, 48, 16, True),
                                                (1, 8, 8, 1, 1, False), (2, 520, 136, 160, 16, False),
                                                (2, 392, 128, 40, 16, True), (1, 384, 128, 320, 16, False)])
def test_conv_xproj_matches_oracle(B, Ls, D, R, N, resume):
    """The conv front fused into x_proj against the oracle's conv front, rounded to bf16, then its
    x_proj.  Bound per output: fp32 accumulation (D 2^-24 sum |W u|), the u elements whose bf16
    rounding the fp32 front end may take the other way (one ulp each, found from the fp64
    values), and the final bf16 rounding."""
    note(f"conv_xproj B={B} L={Ls} D={D} R={R} N={N} resume={resume}")
    prm = I.make_params_distinct(D, 16, seed=D + R)
    g = torch.Generator().manual_seed(B * 1000 + Ls + D + R)
    x = torch.randn(B, D, Ls, generator=g).to(torch.bfloat16)
    w = (torch.randn(R + 2 * N, D, generator=g) / D ** 0.5).to(torch.bfloat16)
    conv0 = torch.randn(B, D, 3, generator=g).to(torch.bfloat16).float() if resume else None
    pd = {k: v.to(DEV) for k, v in prm.items() if v is not None}
    lr, Bm, Cm = L.conv_xproj(x.to(DEV), pd, w.to(DEV), R, None if conv0 is None else conv0.to(DEV))
    torch.cuda.synchronize()
    c0 = None if conv0 is None else conv0.double().numpy()
    u64 = P.conv_silu(x, prm["conv_w"], prm["conv_b"], c0)
    scale = conv_magnitude(x, prm["conv_w"], prm["conv_b"], c0)
    ub = P.to_io(u64, "bf16")
    ref = P.x_proj(ub, w)
    mag = P.x_proj(np.abs(ub), np.abs(w.double().numpy()))
    flips = P.x_proj(bf16_flip_ulps(u64, scale), np.abs(w.double().numpy()))
    b = D * U * mag + flips
    b = b + 2.0 ** -8 * (np.abs(ref) + b)
    got = torch.cat([lr, Bm, Cm], dim=2).double().cpu().numpy()
    err = np.abs(got - ref)
    i = np.unravel_index(int(np.argmax(err - b)), err.shape)
    assert np.all(err <= b), f"{i}: gpu {got[i]!r} ref {ref[i]!r} bound {b[i]:.3e}"
    note(f"conv_xproj: u elements with an open rounding: {int((bf16_flip_ulps(u64, scale) > 0).sum())} "
         f"of {u64.size}")


def test_conv_xproj_no_bias_and_unaligned_outputs():
    """Ragged channels and tokens (D 136 = 2 x 64 + 8, L 264 = 2 x 128 + 8), no conv bias, and
    outputs that are views one element into larger buffers (2-byte aligned only, so written one
    element at a time): equal bit for bit to the call with aligned outputs, which is held to the
    oracle with the bound of test_conv_xproj_matches_oracle."""
    B, Ls, D, R, N = 2, 264, 136, 24, 16
    prm = I.make_params_distinct(D, N, seed=5)
    prm["conv_b"] = None
    g = torch.Generator().manual_seed(55)
    x = torch.randn(B, D, Ls, generator=g).to(torch.bfloat16)
    w = (torch.randn(R + 2 * N, D, generator=g) / D ** 0.5).to(torch.bfloat16)
    pd = {k: v.to(DEV) for k, v in prm.items() if v is not None}
    lr, Bm, Cm = L.conv_xproj(x.to(DEV), pd, w.to(DEV), R)
    bufs = [torch.full((B * Ls * n + 1,), float("nan"), dtype=torch.bfloat16, device=DEV) for n in (R, N, N)]
    views = [bf[1:].view(B, Ls, n) for bf, n in zip(bufs, (R, N, N))]
    L.conv_xproj(x.to(DEV), pd, w.to(DEV), R, lowrank=views[0], Bm=views[1], Cm=views[2])
    torch.cuda.synchronize()
    for a, v, bf in zip((lr, Bm, Cm), views, bufs):
        assert torch.equal(a.view(torch.int16), v.view(torch.int16))
        assert torch.isnan(bf[0])                                   # nothing written before the view
    u64 = P.conv_silu(x, prm["conv_w"], None, None)
    scale = conv_magnitude(x, prm["conv_w"], None, None)
    ub = P.to_io(u64, "bf16")
    ref = P.x_proj(ub, w)
    mag = P.x_proj(np.abs(ub), np.abs(w.double().numpy()))
    flips = P.x_proj(bf16_flip_ulps(u64, scale), np.abs(w.double().numpy()))
    b = D * U * mag + flips
    b = b + 2.0 ** -8 * (np.abs(ref) + b)
    got = torch.cat([lr, Bm, Cm], dim=2).double().cpu().numpy()
    assert np.all(np.abs(got - ref) <= b)


def test_conv_xproj_errors():
    x = torch.randn(1, 16, 64, device=DEV).to(torch.bfloat16)
    prm = {k: v.to(DEV) for k, v in I.make_params(16, 16).items() if v is not None}
    w = torch.randn(40, 16, device=DEV).to(torch.bfloat16)
    with pytest.raises(L.SsmError) as e:
        L.conv_xproj(x.float(), prm, w.float(), 8)       # fp32 io: the fused form is bf16 only
    assert e.value.status == 3
    with pytest.raises(L.SsmError) as e:
        L.conv_xproj(x[:, :, :60].contiguous(), prm, w, 8)   # L not a multiple of 8
    assert e.value.status == 2


def test_conv_xproj_full_size_sampled():
    """The fused conv front + x_proj at the 7B-class layer's size (x [1, 2048, 32768], 288 rows):
    sampled outputs against the oracle's conv front (over the 4 raw inputs each needs) and fp64
    dot products, with the bound of test_conv_xproj_matches_oracle."""
    w8 = I.LAYERS["layer7b"]
    D, Ls, R, N = w8.d_inner, w8.seqlen, w8.dt_rank, w8.d_state
    prm = I.make_params_distinct(D, N)
    pd = {k: v.to(DEV) for k, v in prm.items() if v is not None}
    wall = I.make_proj_weights(w8.d_model, D, R, N, w8.io, device=DEV)["x_all"]
    x = I.make_sequence_device(1, Ls, D, 1, "bf16", device=DEV)["x"]
    lr, Bm, Cm = L.conv_xproj(x, pd, wall, R)
    torch.cuda.synchronize()
    got_all = torch.cat([lr, Bm, Cm], dim=2)[0]                       # [L, 288]
    g = np.random.default_rng(1)
    ts = sorted(set(int(t) for t in g.integers(0, Ls, 24)) | {0, 1, 2, 3, Ls - 1})
    wn = wall.double().cpu().numpy()
    for t in ts:
        lo = max(0, t - 3)
        xs = x[:, :, lo:t + 1].cpu()                                   # [1, D, <= 4]
        u64 = P.conv_silu(xs, prm["conv_w"], prm["conv_b"])[0, :, -1]   # zero history before token 0
        scale = conv_magnitude(xs, prm["conv_w"], prm["conv_b"], None)[0, :, -1]
        ub = P.to_io(u64, "bf16")
        ref = wn @ ub
        mag = np.abs(wn) @ np.abs(ub)
        flips = np.abs(wn) @ bf16_flip_ulps(u64, scale)
        b = D * U * mag + flips
        b = b + 2.0 ** -8 * (np.abs(ref) + b)
        got = got_all[t].double().cpu().numpy()
        assert np.all(np.abs(got - ref) <= b), (t, float(np.max(np.abs(got - ref) - b)))
