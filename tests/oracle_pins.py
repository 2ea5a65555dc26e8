"""Independent pins for the fp64 oracle (importable by the pin tests and the
mutation tests).  Each check takes an oracle ``scan`` callable and raises
AssertionError when the oracle disagrees with something the mathematics fixes.

None of these reuses the oracle's formulas: the brute force sums
exp(A * (cumsum differences)) over all earlier tokens (O(L^2)) with torch's
conv1d / softplus / silu for the front end; the closed form is a geometric
series; the limits reduce to a prefix sum and to a memoryless map; the hand
case was worked on paper (tests/golden/hand_case.json).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
REL = 1e-10


def rand_problem(B, L, D, N, seed, *, resume=False, gate=True, a_scale=1.0, dt_bias=None):
    """Random fp64 problem with per-channel A, D, bias and conv bias (no shared structure)."""
    g = np.random.default_rng(seed)
    p = {
        "x": g.standard_normal((B, D, L)),
        "dt": 0.5 * g.standard_normal((B, D, L)),
        "z": g.standard_normal((B, D, L)) if gate else None,
        "Bm": g.standard_normal((B, L, N)),
        "Cm": g.standard_normal((B, L, N)),
        "A": -a_scale * g.uniform(0.2, 4.0, (D, N)),
        "Dskip": g.uniform(-1.0, 1.5, D),
        "dt_bias": np.log(np.expm1(np.exp(g.uniform(np.log(1e-3), np.log(1e-1), D))))
        if dt_bias is None else np.full(D, float(dt_bias)),
        "conv_w": g.uniform(-0.5, 0.5, (D, 4)),
        "conv_b": g.uniform(-0.2, 0.2, D),
        "h0": g.standard_normal((B, D, N)) if resume else None,
        "conv0": g.standard_normal((B, D, 3)) if resume else None,
    }
    return p


def call(scan, p):
    return scan(p["x"], p["dt"], p["z"], p["Bm"], p["Cm"], p["A"], p["Dskip"], p["dt_bias"],
                p["conv_w"], p["conv_b"], h0=p["h0"], conv0=p["conv0"])


def front_end(p):
    """u = SiLU(causal depthwise conv) and delta = softplus(dt + bias) via torch library routines."""
    T = lambda a: None if a is None else torch.as_tensor(a, dtype=torch.float64)
    x, dt = T(p["x"]), T(p["dt"])
    w, cb, bias = T(p["conv_w"]), T(p["conv_b"]), T(p["dt_bias"])
    B, D, L = x.shape
    hist = T(p["conv0"]) if p["conv0"] is not None else torch.zeros(B, D, 3, dtype=torch.float64)
    xx = torch.cat([hist, x], dim=2)                                # [B, D, L+3]
    v = F.conv1d(xx, w[:, None, :], bias=cb, groups=D)             # cross-correlation: sum_k w_k xx[t+k]
    return F.silu(v), F.softplus(dt + bias[None, :, None]), xx


def brute_force(p):
    """O(L^2) evaluation: h_t[n] = exp(A[n] S_t) h0[n] + sum_{s<=t} exp(A[n](S_t - S_s)) delta_s B_s[n] u_s,
    S_t = delta_0 + ... + delta_t.  Front end through torch library routines."""
    T = lambda a: None if a is None else torch.as_tensor(a, dtype=torch.float64)
    z, Bm, Cm, A, Dk = T(p["z"]), T(p["Bm"]), T(p["Cm"]), T(p["A"]), T(p["Dskip"])
    u, delta, xx = front_end(p)
    B, D, L = u.shape
    S = torch.cumsum(delta, dim=2)                                  # [B, D, L]
    diff = S[:, :, :, None] - S[:, :, None, :]                      # [B, D, t, s]
    causal = torch.tril(torch.ones(L, L, dtype=torch.bool))
    diff = torch.where(causal, diff, torch.zeros_like(diff))
    decay = torch.exp(A[None, :, None, None, :] * diff[..., None])  # [B, D, t, s, N]
    decay = decay * causal[None, None, :, :, None]
    drive = (delta * u)[:, :, :, None] * Bm[:, None, :, :]           # [B, D, s, N]
    h = torch.einsum("bdtsn,bdsn->bdtn", decay, drive)
    if p["h0"] is not None:
        h = h + torch.exp(A[None, :, None, :] * S[..., None]) * T(p["h0"])[:, :, None, :]
    r = torch.einsum("bdtn,btn->bdt", h, Cm) + Dk[None, :, None] * u
    y = r * F.silu(z) if z is not None else r
    conv = xx[:, :, -3:]
    return y.numpy(), h[:, :, -1, :].numpy(), conv.numpy()


def close(a, ref, rel=REL):
    a, ref = np.asarray(a, np.float64), np.asarray(ref, np.float64)
    assert a.shape == ref.shape, (a.shape, ref.shape)
    err = np.abs(a - ref) / (1.0 + np.abs(ref))
    assert np.all(np.isfinite(a)), "non-finite values"
    assert err.max() <= rel, f"max rel err {err.max():.3e} > {rel:.1e} at {np.unravel_index(err.argmax(), err.shape)}"


# ---------------------------------------------------------------------------------------------
def check_brute_force(scan, B=2, L=13, D=3, N=4, seed=1, resume=False, gate=True):
    p = rand_problem(B, L, D, N, seed, resume=resume, gate=gate)
    y, h, c = call(scan, p)
    yb, hb, cb = brute_force(p)
    close(y, yb)
    close(h, hb)
    assert np.array_equal(c, cb), "conv cache must equal the last three raw inputs exactly"


def check_closed_form(scan, L=50, N=5, seed=2, resume=True):
    """Constant delta, A, B and u: h_t = a^{t+1} h0 + delta B u (1 - a^{t+1}) / (1 - a)."""
    g = np.random.default_rng(seed)
    xbar, dtc, bias = 0.7, 0.3, -1.5
    p = {"x": np.full((1, 1, L), xbar), "dt": np.full((1, 1, L), dtc), "z": None,
         "Bm": np.broadcast_to(g.standard_normal(N), (1, L, N)).copy(),
         "Cm": g.standard_normal((1, L, N)), "A": -g.uniform(0.1, 3.0, (1, N)),
         "Dskip": np.array([0.8]), "dt_bias": np.array([bias]),
         "conv_w": np.array([[0.0, 0.0, 0.0, 1.0]]), "conv_b": np.array([0.0]),
         "h0": g.standard_normal((1, 1, N)) if resume else None,
         "conv0": g.standard_normal((1, 1, 3)) if resume else None}
    y, h, _ = call(scan, p)
    ubar = xbar / (1.0 + math.exp(-xbar))
    s = dtc + bias
    delta = math.log1p(math.exp(s))
    A, Bv = p["A"][0], p["Bm"][0, 0]
    t = np.arange(L)[:, None]
    k = delta * A[None, :]
    ht = Bv * delta * ubar * (np.expm1((t + 1) * k) / np.expm1(k))  # [L, N]
    if resume:
        ht = ht + np.exp((t + 1) * k) * p["h0"][0, 0]
    yref = (ht * p["Cm"][0]).sum(1) + 0.8 * ubar
    close(h[0, 0], ht[-1], 1e-12)
    close(y[0, 0], yref, 1e-12)


def check_limits(scan, seed=3):
    """A -> 0: the state is the running sum of delta B u.  A = -1e6: exp underflows to 0 and
    the state forgets everything: y_t = delta_t u_t (C_t . B_t) + D u_t."""
    for A_val, kind in ((-1e-12, "sum"), (-1e6, "memoryless")):
        p = rand_problem(1, 17, 2, 3, seed, gate=False, dt_bias=0.0)
        p["A"] = np.full_like(p["A"], A_val)
        y, h, _ = call(scan, p)
        u, delta, _ = front_end(p)
        u, delta = u[0].numpy(), delta[0].numpy()
        drive = (delta * u)[:, :, None] * p["Bm"][0][None]                  # [D, L, N]
        if kind == "sum":
            hs = np.cumsum(drive, axis=1)
            close(h[0], hs[:, -1], 1e-9)
            yref = (hs * p["Cm"][0][None]).sum(2) + p["Dskip"][:, None] * u
            close(y[0], yref, 1e-9)
        else:
            assert np.all(delta * 1e6 > 800), "limit case needs delta*|A| beyond exp underflow"
            close(h[0], drive[:, -1], 1e-14)
            yref = delta * u * (p["Cm"][0] * p["Bm"][0]).sum(1)[None] + p["Dskip"][:, None] * u
            close(y[0], yref, 1e-14)


def _ev(expr):
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log, "c": math.log(2.0), "l": math.log(3.0)}))


def check_hand_case(scan):
    with open(os.path.join(GOLDEN, "hand_case.json")) as f:
        g = json.load(f)
    i = g["inputs"]
    ev = lambda a: np.vectorize(_ev, otypes=[np.float64])(np.array(a, dtype=object))
    p = {"x": ev(i["x"]).reshape(1, 1, 4), "dt": ev(i["dt"]).reshape(1, 1, 4),
         "z": ev(i["z"]).reshape(1, 1, 4), "Bm": ev(i["Bm"]).reshape(1, 4, 2),
         "Cm": ev(i["Cm"]).reshape(1, 4, 2), "A": ev(i["A"]).reshape(1, 2),
         "Dskip": np.array([_ev(i["Dskip"])]), "dt_bias": np.array([_ev(i["dt_bias"])]),
         "conv_w": ev(i["conv_w"]).reshape(1, 4), "conv_b": np.array([_ev(i["conv_b"])]),
         "h0": None, "conv0": None}
    e = g["expected"]
    r, gate = ev(e["r"]), ev(e["gate"])
    y, h, c = call(scan, p)
    close(y[0, 0], r * gate, 1e-14)
    close(h[0, 0], ev(e["h_final"]), 1e-14)
    assert np.array_equal(c[0, 0], ev(e["conv_final"]))
    p["z"] = None
    y2, _, _ = call(scan, p)
    close(y2[0, 0], r, 1e-14)


def check_conv_special(scan, seed=4):
    """w = (0,0,0,1): u = silu(x).  w = (1,0,0,0): u_t = silu(x_{t-3}), zero for t < 3.
    Read through the memoryless limit (A = -1e6, dt_bias = 0, N = 1, B = C = 1, D = 0):
    y_t = delta_t u_t."""
    p = rand_problem(1, 9, 1, 1, seed, gate=False, dt_bias=0.0)
    p.update(A=np.array([[-1e6]]), Bm=np.ones((1, 9, 1)), Cm=np.ones((1, 9, 1)),
             Dskip=np.array([0.0]), conv_b=np.array([0.0]))
    s = p["dt"][0, 0]
    delta = torch.nn.functional.softplus(torch.as_tensor(s)).numpy()
    x = p["x"][0, 0]
    silu = lambda a: torch.nn.functional.silu(torch.as_tensor(a)).numpy()
    p["conv_w"] = np.array([[0.0, 0.0, 0.0, 1.0]])
    y, _, _ = call(scan, p)
    close(y[0, 0], delta * silu(x), 1e-13)
    p["conv_w"] = np.array([[1.0, 0.0, 0.0, 0.0]])
    y, _, _ = call(scan, p)
    shifted = np.concatenate([np.zeros(3), x[:-3]])
    close(y[0, 0], delta * silu(shifted), 1e-13)


def check_conv_cache(scan, seed=5):
    """conv cache = raw inputs x[L-3..L-1], oldest first, zero-filled (or history) when L < 3."""
    for L in (1, 2, 3, 4, 7):
        for resume in (False, True):
            p = rand_problem(2, L, 3, 2, seed + L, resume=resume)
            _, _, c = call(scan, p)
            hist = p["conv0"] if resume else np.zeros((2, 3, 3))
            want = np.concatenate([hist, p["x"]], 2)[:, :, -3:]
            assert np.array_equal(c, want), f"conv cache wrong at L={L} resume={resume}"


def check_prefill_then_decode(scan, seed=6, L1=11, L2=6):
    """Invariant of state caching: prefill(L1) then L2 single-token steps from the cache
    equals prefill(L1 + L2) (bitwise: the oracle runs the same operations in the same order)."""
    p = rand_problem(2, L1 + L2, 3, 4, seed)
    y, h, c = call(scan, p)
    q = dict(p)
    for k in ("x", "dt", "z"):
        q[k] = p[k][:, :, :L1]
    for k in ("Bm", "Cm"):
        q[k] = p[k][:, :L1]
    y1, hc, cc = call(scan, q)
    assert np.array_equal(y1, y[:, :, :L1])
    for t in range(L1, L1 + L2):
        r = dict(p)
        for k in ("x", "dt", "z"):
            r[k] = p[k][:, :, t:t + 1]
        for k in ("Bm", "Cm"):
            r[k] = p[k][:, t:t + 1]
        r["h0"], r["conv0"] = hc, cc
        yt, hc, cc = call(scan, r)
        assert np.array_equal(yt[:, :, 0], y[:, :, t]), f"decode step {t} differs from prefill"
    assert np.array_equal(hc, h) and np.array_equal(cc, c)


def check_channel_slices(scan, seed=7):
    """Channel locality: disjoint channel slices run alone equal the full run (bitwise);
    so do single batch rows."""
    p = rand_problem(3, 10, 7, 4, seed, resume=True)
    y, h, c = call(scan, p)
    for lo, hi in ((0, 3), (3, 4), (4, 7)):
        q = dict(p)
        for k in ("x", "dt", "z", "h0", "conv0"):
            q[k] = p[k][:, lo:hi]
        for k in ("A", "Dskip", "dt_bias", "conv_w", "conv_b"):
            q[k] = p[k][lo:hi]
        ys, hs, cs = call(scan, q)
        assert np.array_equal(ys, y[:, lo:hi]) and np.array_equal(hs, h[:, lo:hi]) and np.array_equal(cs, c[:, lo:hi])
    for b in range(3):
        q = dict(p)
        for k in ("x", "dt", "z", "Bm", "Cm", "h0", "conv0"):
            q[k] = p[k][b:b + 1]
        ys, hs, cs = call(scan, q)
        assert np.array_equal(ys, y[b:b + 1]) and np.array_equal(hs, h[b:b + 1])


def check_pow2_scaling(scan, seed=8):
    """With Dskip = 0: C x 2 doubles y; B x 2 doubles h and y -- exactly, in binary floating point."""
    p = rand_problem(1, 12, 3, 4, seed)
    p["Dskip"] = np.zeros(3)
    y, h, _ = call(scan, p)
    q = dict(p, Cm=2.0 * p["Cm"])
    y2, h2, _ = call(scan, q)
    assert np.array_equal(y2, 2.0 * y) and np.array_equal(h2, h)
    q = dict(p, Bm=2.0 * p["Bm"])
    y3, h3, _ = call(scan, q)
    assert np.array_equal(h3, 2.0 * h) and np.array_equal(y3, 2.0 * y)


ALL_CHECKS = {
    "brute_force": lambda s: [check_brute_force(s, **kw) for kw in (
        dict(), dict(resume=True), dict(gate=False), dict(B=1, L=1, D=1, N=1), dict(B=1, L=2, D=2, N=16),
        dict(B=2, L=5, D=3, N=1))],
    "closed_form": lambda s: [check_closed_form(s, resume=r) for r in (False, True)],
    "limits": check_limits,
    "hand_case": check_hand_case,
    "conv_special": check_conv_special,
    "conv_cache": check_conv_cache,
    "prefill_then_decode": check_prefill_then_decode,
    "channel_slices": check_channel_slices,
    "pow2_scaling": check_pow2_scaling,
}
