"""Independent pins for the projection / conv-front oracle (oracle/proj.py), importable by
the pin tests and the mutation tests.  Each check takes a module with in_proj, x_proj,
dt_proj, out_proj and conv_silu and raises AssertionError on a disagreement.

None of these reuses the oracle's code: products are checked against triple loops in plain
Python on small sizes whose dimensions are all distinct (so a transposed operand or output
cannot go unnoticed), against identity weights, and by linearity; the conv front against
torch's conv1d in fp64 and against its tap special cases and the resume invariance.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

B, L, DM, D, J, R = 2, 3, 5, 4, 6, 7   # all distinct


def _rng(seed):
    return np.random.default_rng(seed)


def check_in_proj_brute(P):
    g = _rng(1)
    h, w = g.standard_normal((B, L, DM)), g.standard_normal((D, DM))
    out = P.in_proj(h, w)
    assert out.shape == (B, D, L), out.shape
    for b in range(B):
        for c in range(D):
            for t in range(L):
                ref = sum(float(w[c, k]) * float(h[b, t, k]) for k in range(DM))
                assert abs(out[b, c, t] - ref) <= 1e-12 * (1 + abs(ref)), (b, c, t)


def check_x_proj_brute(P):
    g = _rng(2)
    u, w = g.standard_normal((B, D, L)), g.standard_normal((J, D))
    out = P.x_proj(u, w)
    assert out.shape == (B, L, J), out.shape
    for b in range(B):
        for t in range(L):
            for j in range(J):
                ref = sum(float(w[j, c]) * float(u[b, c, t]) for c in range(D))
                assert abs(out[b, t, j] - ref) <= 1e-12 * (1 + abs(ref)), (b, t, j)


def check_dt_proj_brute(P):
    g = _rng(3)
    lr, w = g.standard_normal((B, L, R)), g.standard_normal((D, R))
    out = P.dt_proj(lr, w)
    assert out.shape == (B, D, L), out.shape
    for b in range(B):
        for c in range(D):
            for t in range(L):
                ref = sum(float(w[c, r]) * float(lr[b, t, r]) for r in range(R))
                assert abs(out[b, c, t] - ref) <= 1e-12 * (1 + abs(ref)), (b, c, t)


def check_out_proj_brute(P):
    g = _rng(4)
    y, w = g.standard_normal((B, D, L)), g.standard_normal((DM, D))
    out = P.out_proj(y, w)
    assert out.shape == (B, L, DM), out.shape
    for b in range(B):
        for t in range(L):
            for m in range(DM):
                ref = sum(float(w[m, c]) * float(y[b, c, t]) for c in range(D))
                assert abs(out[b, t, m] - ref) <= 1e-12 * (1 + abs(ref)), (b, t, m)


def check_identity_weights(P):
    """W = I: in_proj is the channel-major transpose of hidden; out_proj its inverse."""
    g = _rng(5)
    h = g.standard_normal((B, L, D))
    x = P.in_proj(h, np.eye(D))
    assert np.array_equal(x, np.transpose(h, (0, 2, 1)))
    assert np.array_equal(P.out_proj(x, np.eye(D)), h)
    assert np.array_equal(P.x_proj(x, np.eye(D)), h)
    assert np.array_equal(P.dt_proj(h, np.eye(D)), x)


def check_linearity(P):
    """Doubling the weights doubles every output exactly (powers of two are exact)."""
    g = _rng(6)
    h, w = g.standard_normal((B, L, DM)), g.standard_normal((D, DM))
    assert np.array_equal(P.in_proj(h, 2 * w), 2 * P.in_proj(h, w))
    u, w2 = g.standard_normal((B, D, L)), g.standard_normal((J, D))
    assert np.array_equal(P.x_proj(2 * u, w2), 2 * P.x_proj(u, w2))


def _torch_conv_silu(x, w, b, conv0):
    xt = torch.from_numpy(np.asarray(x, np.float64))
    Bn, Dn, Ln = xt.shape
    hist = torch.zeros(Bn, Dn, 3, dtype=torch.float64) if conv0 is None else torch.from_numpy(np.asarray(conv0))
    full = torch.cat([hist, xt], dim=2)                      # history then the tokens
    wt = torch.from_numpy(np.asarray(w, np.float64)).unsqueeze(1)   # [D, 1, 4]
    bt = None if b is None else torch.from_numpy(np.asarray(b, np.float64))
    v = F.conv1d(full, wt, bt, groups=Dn)                    # valid conv: output t uses full[t..t+3]
    return F.silu(v).numpy()


def check_conv_silu_torch(P):
    g = _rng(7)
    for resume in (False, True):
        x = g.standard_normal((2, 6, 11))
        w = g.uniform(-0.5, 0.5, (6, 4))
        b = g.standard_normal(6)
        c0 = g.standard_normal((2, 6, 3)) if resume else None
        u = P.conv_silu(x, w, b, c0)
        ref = _torch_conv_silu(x, w, b, c0)
        assert u.shape == ref.shape and np.allclose(u, ref, rtol=1e-13, atol=1e-14), np.abs(u - ref).max()


def check_conv_taps(P):
    g = _rng(8)
    x = g.standard_normal((1, 3, 9))
    last = np.tile([0.0, 0.0, 0.0, 1.0], (3, 1))
    first = np.tile([1.0, 0.0, 0.0, 0.0], (3, 1))
    silu = lambda v: v / (1 + np.exp(-v))
    assert np.allclose(P.conv_silu(x, last), silu(x), rtol=1e-15, atol=0)
    shifted = np.concatenate([np.zeros((1, 3, 3)), x[:, :, :-3]], axis=2)
    assert np.allclose(P.conv_silu(x, first), silu(shifted), rtol=1e-15, atol=0)


def check_conv_resume(P):
    """Running tokens [L1, L) with the last three raw inputs before L1 as history equals the
    tail of the full run, bitwise."""
    g = _rng(9)
    x = g.standard_normal((2, 4, 13))
    w = g.uniform(-0.5, 0.5, (4, 4))
    b = g.standard_normal(4)
    full = P.conv_silu(x, w, b)
    for L1 in (1, 3, 7):
        hist = np.concatenate([np.zeros((2, 4, 3)), x], axis=2)[:, :, L1:L1 + 3]
        tail = P.conv_silu(x[:, :, L1:], w, b, hist)
        assert np.array_equal(tail, full[:, :, L1:]), L1


def _small_layer(seed):
    """A small random layer (all sizes distinct): hidden [B, L1 + 1, d_model], weights, and
    per-channel scan parameters, as plain arrays."""
    g = _rng(seed)
    Bs, L1, dm, d, r, n = 2, 9, 12, 8, 5, 4
    w = {"in_x": g.standard_normal((d, dm)) / dm ** 0.5, "in_z": g.standard_normal((d, dm)) / dm ** 0.5,
         "x_dt": g.standard_normal((r, d)) / d ** 0.5, "x_B": g.standard_normal((n, d)) / d ** 0.5,
         "x_C": g.standard_normal((n, d)) / d ** 0.5, "dt": 0.5 * g.standard_normal((d, r)) / r ** 0.5,
         "out": g.standard_normal((dm, d)) / d ** 0.5}
    prm = {"A": -np.exp(g.uniform(-2, 2, (d, n))), "Dskip": g.uniform(0.25, 2.0, d),
           "dt_bias": np.log(np.expm1(np.exp(g.uniform(np.log(1e-2), 0.0, d)))),
           "conv_w": g.uniform(-0.5, 0.5, (d, 4)), "conv_b": g.uniform(-0.6, 0.6, d)}
    return g.standard_normal((Bs, L1 + 1, dm)), w, prm, L1


def check_layer_decode_is_next_token(P):
    """The layer's caching invariant (page 1, Methodology item 3): decoding token L1 from the
    cache a prefill of L1 tokens leaves gives what a prefill of L1 + 1 tokens gives at its last
    token -- the out partial, and the final state and conv window -- bit for bit (every stage
    computes each token's value by the same operations in both)."""
    hidden, w, prm, L1 = _small_layer(10)
    for io in ("f32", "bf16"):
        out_full, h_full, c_full = P.layer_prefill(hidden, w, prm, io)
        _, h1, c1 = P.layer_prefill(hidden[:, :L1], w, prm, io)
        out_t, _, h2, c2 = P.layer_decode_step(hidden[:, L1], w, prm, h1, c1, io)
        assert np.array_equal(out_t, out_full[:, L1]), (io, np.abs(out_t - out_full[:, L1]).max())
        assert np.array_equal(h2, h_full) and np.array_equal(c2, c_full), io


ALL_CHECKS = {
    "in_proj_brute": check_in_proj_brute,
    "x_proj_brute": check_x_proj_brute,
    "dt_proj_brute": check_dt_proj_brute,
    "out_proj_brute": check_out_proj_brute,
    "identity_weights": check_identity_weights,
    "linearity": check_linearity,
    "conv_silu_torch": check_conv_silu_torch,
    "conv_taps": check_conv_taps,
    "conv_resume": check_conv_resume,
    "layer_decode_is_next_token": check_layer_decode_is_next_token,
}
