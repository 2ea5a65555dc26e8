"""Calls too large for one kernel launch (needs an MI355X; a few GB of device memory each).

The scan splits a call into launches over batch rows, each of at most 2^31 work-items at 64 per
channel: with d_inner 2048 one launch holds 16256 rows, and these calls have more.  Rows on both
sides of every split are checked against the oracle, and the prefill rows also bit for bit
against the same row run alone.  The conv front and the int8 quantizer stride over a capped grid
(2^20 workgroups); their calls here exceed the cap, and sampled outputs past it are checked
against their oracles."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_causal_amd as ssm
from oracle import codec as QC
from oracle import proj as P
from selective_state_space_causal_amd import inputs as I
from tests.gpu_common import DEV, TAU, assert_bitwise, assert_close, dev, f64, note

pytestmark = pytest.mark.gpu

D = 2048
ROWS_PER_LAUNCH = (1 << 31) // (64 * (D + 16))   # 16256
B = 2 * ROWS_PER_LAUNCH + 37                      # three launches
CHECK = [0, ROWS_PER_LAUNCH - 1, ROWS_PER_LAUNCH, ROWS_PER_LAUNCH + 1, 2 * ROWS_PER_LAUNCH, B - 1]


def host_row(seq, b, n=None):
    return {k: (None if v is None else (v[b:b + 1, :, :n] if k in ("x", "dt", "z") else v[b:b + 1, :n]).cpu())
            for k, v in seq.items()}


def row_oracle(seq, prm, b, n=None, h0=None, conv0=None):
    r = host_row(seq, b, n)
    y, h, c = oracle.scan(r["x"], r["dt"], r["z"], r["Bm"], r["Cm"], prm["A"], prm["Dskip"], prm["dt_bias"],
                          prm["conv_w"], prm.get("conv_b"), h0=h0, conv0=conv0)
    return y[0], h[0], c[0]


@pytest.mark.parametrize("N", [16, 4])
def test_prefill_split_over_batch_rows(N):
    L = 8
    note(f"large prefill B={B} D={D} L={L} N={N}")
    prm = I.make_params_distinct(D, N, seed=61)
    seq = I.make_sequence_device(B, L, D, N, "bf16", seed=61, device=DEV)
    pd = dev(prm)
    y, h, c = ssm.prefill(seq["x"], seq["dt"], seq["z"], seq["Bm"], seq["Cm"], pd)
    torch.cuda.synchronize()
    for b in CHECK:
        yr, hr, cr = row_oracle(seq, prm, b)
        assert_close(y[b], yr, TAU["bf16"], f"row {b} y")
        assert_close(h[b], hr, TAU["bf16"], f"row {b} h")
        assert_bitwise(c[b], cr, f"row {b} conv")
        one = {k: v[b:b + 1].contiguous() for k, v in seq.items()}
        yb, hb, cb = ssm.prefill(one["x"], one["dt"], one["z"], one["Bm"], one["Cm"], pd)
        torch.cuda.synchronize()
        assert torch.equal(yb[0].view(torch.int16), y[b].view(torch.int16)), b
        assert torch.equal(hb[0], h[b]) and torch.equal(cb[0], c[b]), b


@pytest.mark.parametrize("N", [16, 4])
def test_decode_split_over_batch_rows(N):
    note(f"large decode B={B} D={D} N={N}")
    prm = I.make_params_distinct(D, N, seed=62)
    g = torch.Generator(device=DEV).manual_seed(62)
    h = torch.randn(B, D, N, generator=g, device=DEV)
    c = torch.randn(B, D, 3, generator=g, device=DEV).to(torch.bfloat16).float()
    tok = {k: v[..., 0].contiguous() if k in ("x", "dt", "z") else v[:, 0].contiguous()
           for k, v in I.make_sequence_device(B, 1, D, N, "bf16", seed=63, device=DEV).items()}
    h_in = {b: f64(h[b]) for b in CHECK}
    c_in = {b: f64(c[b]) for b in CHECK}
    y = ssm.decode_step(tok["x"], tok["dt"], tok["z"], tok["Bm"], tok["Cm"], dev(prm), h, c)
    torch.cuda.synchronize()
    for b in CHECK:
        tb = {k: v[b:b + 1].cpu() for k, v in tok.items()}
        yr, hr, cr = oracle.decode_step(tb, prm, h_in[b][None], c_in[b][None])
        assert_close(y[b], yr[0], TAU["bf16"], f"row {b} y")
        assert_close(h[b], hr[0], TAU["bf16"], f"row {b} h")
        assert_bitwise(c[b], cr[0], f"row {b} conv")


def test_prefill_pool_split_over_batch_rows():
    """The pool form: each launch takes its rows' slots and lengths; the pool is shared."""
    L, N = 16, 16
    note(f"large prefill_pool B={B} D={D} L={L}")
    prm = I.make_params_distinct(D, N, seed=64)
    seq = I.make_sequence_device(B, L, D, N, "bf16", seed=64, device=DEV)
    g = torch.Generator().manual_seed(64)
    S = B + 3
    slots = torch.randperm(S, generator=g)[:B].to(torch.int32)
    lens = torch.randint(0, L + 1, (B,), generator=g, dtype=torch.int32)
    hp = torch.zeros(S, D, N, device=DEV)
    cp = torch.zeros(S, D, 3, device=DEV)
    y = ssm.prefill_pool(seq["x"], seq["dt"], seq["z"], seq["Bm"], seq["Cm"], dev(prm), slots.to(DEV), hp, cp,
                         seqlens=lens.to(DEV))
    torch.cuda.synchronize()
    for b in CHECK:
        n, s = int(lens[b]), int(slots[b])
        if n == 0:
            assert torch.all(hp[s] == 0) and torch.all(cp[s] == 0), b
            continue
        yr, hr, cr = row_oracle(seq, prm, b, n)
        assert_close(y[b, :, :n], yr, TAU["bf16"], f"row {b} y")
        assert_close(hp[s], hr, TAU["bf16"], f"row {b} h")
        assert_bitwise(cp[s], cr, f"row {b} conv")


def test_conv_front_past_the_grid_cap():
    """2^31 + 2^16 tokens in 8-token lanes: more lanes than 2^20 workgroups of 256 hold."""
    Bc, Dc, Lc = 1, 4096, (1 << 19) + 16
    note(f"large conv_silu B={Bc} D={Dc} L={Lc}")
    prm = I.make_params_distinct(Dc, 16, seed=65)
    x = I.make_sequence_device(Bc, Lc, Dc, 1, "bf16", seed=65, device=DEV)["x"]
    u = ssm.conv_silu(x, dev(prm))
    torch.cuda.synchronize()
    for c in (0, 1234, 2047, 2048, Dc - 1):   # rows in the first and the last grid-stride passes
        for t0 in (0, Lc // 2, Lc - 40):
            xs = x[0:1, c:c + 1, max(0, t0 - 3):t0 + 40].cpu()
            hist = None if t0 == 0 else xs[:, :, :3].double().numpy()
            cb = prm.get("conv_b")
            ref = P.conv_silu(xs[:, :, 0 if t0 == 0 else 3:], prm["conv_w"][c:c + 1],
                              None if cb is None else cb[c:c + 1], hist)
            got = f64(u[0:1, c:c + 1, t0:t0 + 40])
            tol = 2.0 ** -8 * np.abs(ref) + 1e-6 * (1 + np.abs(ref))
            assert np.all(np.abs(got - ref) <= tol), (c, t0)


def test_quantize_past_the_grid_cap():
    """2^31 + 3000 bf16 values: more 2048-element tiles than the 2^20-workgroup grid."""
    n, block = (1 << 31) + 3000, 128
    note(f"large q8_quantize n={n}")
    g = torch.Generator(device=DEV).manual_seed(66)
    x = torch.randn(n, generator=g, device=DEV).to(torch.bfloat16)
    q, sc = ssm.q8_quantize(x, block)
    torch.cuda.synchronize()
    for e0 in (0, (1 << 31) - 2048, 1 << 31, n - (n % block)):
        e1 = min(n, e0 + 4 * block)
        qr, sr = QC.quantize(x[e0:e1].float().cpu().numpy(), block)
        assert np.array_equal(q[e0:e1].cpu().numpy(), qr), e0
        got = sc[e0 // block:e0 // block + len(sr)].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), sr.view(np.uint32)), e0


def _decode_rows_case(Bn, Dn, check, seed):
    """One decode step over Bn batch rows of Dn channels (tokens drawn on the device), checked on
    whole rows against the oracle.  The decode kernel finds each quad's batch row and channel with
    a multiply-shift division by Dn; these cases put large quotients (many rows per launch) and
    large, odd divisors through it, on both sides of a launch split."""
    N = 16
    note(f"decode rows B={Bn} D={Dn} (launch split every {(1 << 31) // (64 * (Dn + 16))} rows)")
    prm = I.make_params_distinct(Dn, N, seed=seed)
    g = torch.Generator(device=DEV).manual_seed(seed)
    bf = torch.bfloat16
    tok = {"x": torch.randn(Bn, Dn, generator=g, device=DEV).to(bf),
           "dt": (0.5 * torch.randn(Bn, Dn, generator=g, device=DEV)).to(bf),
           "z": torch.randn(Bn, Dn, generator=g, device=DEV).to(bf),
           "Bm": torch.randn(Bn, N, generator=g, device=DEV).to(bf),
           "Cm": torch.randn(Bn, N, generator=g, device=DEV).to(bf)}
    h = torch.randn(Bn, Dn, N, generator=g, device=DEV)
    c = torch.randn(Bn, Dn, 3, generator=g, device=DEV).to(bf).float()
    h_in = {b: f64(h[b]) for b in check}
    c_in = {b: f64(c[b]) for b in check}
    y = ssm.decode_step(tok["x"], tok["dt"], tok["z"], tok["Bm"], tok["Cm"], dev(prm), h, c)
    torch.cuda.synchronize()
    for b in check:
        tb = {k: v[b:b + 1].cpu() for k, v in tok.items()}
        yr, hr, cr = oracle.decode_step(tb, prm, h_in[b][None], c_in[b][None])
        assert_close(y[b], yr[0], TAU["bf16"], f"row {b} y")
        assert_close(h[b], hr[0], TAU["bf16"], f"row {b} h")
        assert_bitwise(c[b], cr[0], f"row {b} conv")


def test_decode_large_odd_divisor():
    Dn = (1 << 20) + 1
    per = (1 << 31) // (64 * (Dn + 16))  # 31 rows per launch
    _decode_rows_case(40, Dn, [0, 1, per - 1, per, per + 1, 39], seed=64)


def test_decode_small_divisor_many_rows():
    Dn = 3
    per = (1 << 31) // (64 * (Dn + 16))  # 1766022 rows per launch
    Bn = per + 233979                      # two launches
    _decode_rows_case(Bn, Dn, [0, 1, 777777, per - 1, per, per + 1, Bn - 1], seed=65)
