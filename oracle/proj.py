"""Channel-sliced projections either side of the scan, and the conv front on its own:
plain CPU oracle (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the GPU library.

What it follows: "Scaling State-Space Models on Multiple GPUs with Tensor Parallelism"
(euno.news summary of arXiv 2602.21144), Methodology item 1: the mixer's packed weight
tensor (its long-range projections and its local mixing kernels) is split across GPUs along
the feature dimension, as in Transformer tensor parallelism, while item 2 keeps the
recurrence local.  One GPU therefore holds a column shard of the input projection (its own
channels of x and z), the rows of the projection that makes the step sizes and B / C that
read its channels (a partial sum over channels), the step-size projection of its own
channels, and a row shard of the output projection (a partial sum that the ranks add).
The pages do not write these maps; the Mamba mixer's (Gu & Dao, 2023) are used, in this
library's layouts:
  in_proj   out[b, c, t] = sum_k W[c, k] hidden[b, t, k]    W [D, d_model], out [B, D, L]
  x_proj    out[b, t, j] = sum_c W[j, c] u[b, c, t]         W [J, D],       out [B, L, J]
  dt_proj   out[b, c, t] = sum_r W[c, r] lowrank[b, t, r]   W [D, R],       out [B, D, L]
  out_proj  out[b, t, m] = sum_c W[m, c] y[b, c, t]         W [d_model, D], out [B, L, d_model]
  conv_silu u[b, c, t] = silu(conv_b[c] + sum_k conv_w[c, k] xi[b, c, t - 3 + k])
(xi = the raw x, with history xi[-3..-1] = conv0 or zeros).  Each function takes the same
io bits the GPU reads (widened exactly to fp64) and returns fp64.  Each projection is one
library matrix product (numpy einsum) with no blocking or reordering.

Pins: tests/proj_pins.py (torch conv1d in fp64, tap special cases, resume invariance, brute
force triple loops on small sizes with all dimensions distinct, identity weights,
linearity), with planted mistakes in tests/test_proj_mutants.py.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor (any dtype, any device)
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def in_proj(hidden, w) -> np.ndarray:
    """hidden [B, L, d_model], W [D, d_model] -> [B, D, L]."""
    return np.einsum("blk,ck->bcl", _f64(hidden), _f64(w))


def x_proj(u, w) -> np.ndarray:
    """u [B, D, L], W [J, D] -> [B, L, J] (this slice's partial sum over channels)."""
    return np.einsum("bcl,jc->blj", _f64(u), _f64(w))


def dt_proj(lowrank, w) -> np.ndarray:
    """lowrank [B, L, R], W [D, R] -> [B, D, L]."""
    return np.einsum("blr,cr->bcl", _f64(lowrank), _f64(w))


def out_proj(y, w) -> np.ndarray:
    """y [B, D, L], W [d_model, D] -> [B, L, d_model] (this slice's partial sum)."""
    return np.einsum("bcl,mc->blm", _f64(y), _f64(w))


def conv_silu(x, conv_w, conv_b=None, conv0: Optional[np.ndarray] = None) -> np.ndarray:
    """x [B, D, L], conv_w [D, 4], conv_b [D] or None, conv0 [B, D, 3] or None -> u [B, D, L]."""
    x = _f64(x)
    B, D, L = x.shape
    w = _f64(conv_w)
    hist = np.zeros((B, D, 3)) if conv0 is None else _f64(conv0)
    xi = np.concatenate([hist, x], axis=2)          # xi[..., s] = raw input at token s - 3
    v = np.zeros((B, D, L)) if conv_b is None else np.broadcast_to(_f64(conv_b)[None, :, None], (B, D, L)).copy()
    for k in range(4):                               # tap k multiplies the input at t - 3 + k
        v = v + w[None, :, k, None] * xi[:, :, k:k + L]
    with np.errstate(over="ignore"):                 # e^-v = inf gives the limit -0
        return v / (1.0 + np.exp(-v))


def to_io(a, io: str) -> np.ndarray:
    """Round fp64 values to the io dtype the GPU stores a tensor in (bf16: through fp32, each
    step round to nearest even), returned widened to fp64."""
    import torch  # test infrastructure; torch's casts are round-to-nearest-even

    t = torch.from_numpy(np.asarray(a, dtype=np.float64)).to(torch.float32)
    if io == "bf16":
        t = t.to(torch.bfloat16)
    return t.double().numpy()


def layer_prefill(hidden, w: dict, params: dict, io: str = "bf16", nthreads: int = 1, out_io: bool = True):
    """One rank's mixer layer over a prompt, as the library composes it: in_proj (x, z),
    conv front, x_proj (low-rank step input, B, C), dt_proj, the scan (the C oracle), and
    out_proj, whose partial is rounded to the io dtype when out_io (else kept exact); every
    intermediate tensor the GPU stores in the io dtype is rounded to it here at the same
    point.  Returns (out [B, L, d_model] fp64, h, conv)."""
    from . import prefill as scan_prefill  # the fp64 C oracle of the scan

    x = to_io(in_proj(hidden, w["in_x"]), io)
    z = to_io(in_proj(hidden, w["in_z"]), io)
    u = to_io(conv_silu(x, params["conv_w"], params.get("conv_b")), io)
    lowrank = to_io(x_proj(u, w["x_dt"]), io)
    Bm = to_io(x_proj(u, w["x_B"]), io)
    Cm = to_io(x_proj(u, w["x_C"]), io)
    dt = to_io(dt_proj(lowrank, w["dt"]), io)
    y, h, c = scan_prefill({"x": x, "dt": dt, "z": z, "Bm": Bm, "Cm": Cm},
                           {k: _f64(v) for k, v in params.items() if v is not None}, nthreads=nthreads)
    y = to_io(y, io)
    out = out_proj(y, w["out"])
    return (to_io(out, io) if out_io else out), h, c


def layer_decode_step(hidden_t, w: dict, params: dict, h, conv, io: str = "bf16", out_io: bool = True):
    """One decoded token through one rank's mixer layer, as the library composes it: in_proj
    (x_t, z_t), the conv front from the conv cache, x_proj (low-rank step input, B_t, C_t),
    dt_proj, the decode step of the scan (the C oracle, resumed from h and conv), and out_proj;
    every intermediate the GPU stores in the io dtype is rounded to it at the same point.
    hidden_t [B, d_model]; h [B, D, N]; conv [B, D, 3].  Returns (out [B, d_model] fp64,
    y [B, D], h', conv')."""
    from . import decode_step as scan_decode  # the fp64 C oracle of the scan

    hid = _f64(hidden_t)[:, None, :]                                   # [B, 1, d_model]
    x = to_io(in_proj(hid, w["in_x"]), io)                             # [B, D, 1]
    z = to_io(in_proj(hid, w["in_z"]), io)
    u = to_io(conv_silu(x, params["conv_w"], params.get("conv_b"), _f64(conv)), io)
    lowrank = to_io(x_proj(u, w["x_dt"]), io)                          # [B, 1, R]
    Bm = to_io(x_proj(u, w["x_B"]), io)
    Cm = to_io(x_proj(u, w["x_C"]), io)
    dt = to_io(dt_proj(lowrank, w["dt"]), io)                          # [B, D, 1]
    tok = {"x": x[..., 0], "dt": dt[..., 0], "z": z[..., 0], "Bm": Bm[:, 0], "Cm": Cm[:, 0]}
    y, h2, c2 = scan_decode(tok, {k: _f64(v) for k, v in params.items() if v is not None}, _f64(h), _f64(conv))
    y = to_io(y, io)
    out = out_proj(y[..., None], w["out"])[:, 0]
    return (to_io(out, io) if out_io else out), y, h2, c2
