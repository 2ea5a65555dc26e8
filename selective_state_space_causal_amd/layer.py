"""One rank's slice of a selective-SSM mixer layer over a prompt, composed from the library's
C-ABI calls (argument marshalling only; every step runs in the library's kernels or in its
hipBLASLt GEMMs):

  x, z    = in_proj (column shard)            [B, L, d_model] -> [B, D, L] each
  u       = conv + SiLU front                 [B, D, L]
  r, B, C = x_proj rows reading these channels [B, D, L] -> [B, L, R], [B, L, N], [B, L, N]
  dt      = dt_proj                           [B, L, R] -> [B, D, L]
  y, h, c = ssm_prefill                       (the scan; leaves the h / conv cache)
  out     = out_proj (row shard)              [B, D, L] -> [B, L, d_model], a partial sum

"Scaling State-Space Models on Multiple GPUs with Tensor Parallelism" (euno.news summary of
arXiv 2602.21144), Methodology items 1-2.  With more than one rank, x_proj's outputs and out
are partial sums that the ranks add (all-reduces outside this build); on one GPU the slice's
partials are used as they are.

in_proj's shard is one [2D, d_model] weight whose first D rows make x and last D rows make z
(the mixer's packed input projection).  With one batch row, one GEMM writes [1, 2D, L] and x
and z are its two halves, each already a contiguous [1, D, L] tensor; otherwise the two halves
of the weight run as two GEMMs.  x_proj's rows are stacked likewise ([R + 2N, D]: low-rank, B,
C); for bf16 with D and L multiples of 8, the conv front and x_proj run as one fused kernel
(ssm_conv_xproj) and u is never stored; otherwise u is materialised and x_proj runs as three
GEMMs.  out is written in the io dtype by default (the partial that the 8-bit all-reduce codec
then quantizes); out_dtype=torch.float32 keeps it in fp32.
"""
from __future__ import annotations

import torch

from . import _lib

CONV_W = 4


def _stacked_in_proj(hidden, weights) -> bool:
    """True when one GEMM can write x and z: a stacked weight, one batch row, and z's half
    starting on a 16-byte boundary."""
    if "in_xz" not in weights or hidden.shape[0] != 1:
        return False
    D, L = weights["in_xz"].shape[0] // 2, hidden.shape[1]
    return (D * L * hidden.element_size()) % 16 == 0


def _fused_conv_xproj(hidden, weights) -> bool:
    """True when the conv front and x_proj can run as one kernel: the stacked x_proj weight,
    bf16, and d_inner and seqlen multiples of 8."""
    D, L = weights["in_x"].shape[0], hidden.shape[1]
    return "x_all" in weights and hidden.dtype == torch.bfloat16 and D % 8 == 0 and L % 8 == 0


def alloc_buffers(hidden, weights: dict, d_state: int, out_dtype=None) -> dict:
    """Every tensor the layer writes, on hidden's device."""
    B, L, DM = hidden.shape
    D = weights["in_x"].shape[0]
    R = weights["x_dt"].shape[0]
    dev, dt = hidden.device, hidden.dtype
    bufs = {}
    if _stacked_in_proj(hidden, weights):
        bufs["xz"] = torch.empty(B, 2 * D, L, dtype=dt, device=dev)
        bufs["x"], bufs["z"] = bufs["xz"][:, :D], bufs["xz"][:, D:]
    else:
        bufs["x"] = torch.empty(B, D, L, dtype=dt, device=dev)
        bufs["z"] = torch.empty_like(bufs["x"])
    for k in ("dt", "y") if _fused_conv_xproj(hidden, weights) else ("u", "dt", "y"):
        bufs[k] = torch.empty(B, D, L, dtype=dt, device=dev)
    bufs["lowrank"] = torch.empty(B, L, R, dtype=dt, device=dev)
    bufs["Bm"] = torch.empty(B, L, d_state, dtype=dt, device=dev)
    bufs["Cm"] = torch.empty(B, L, d_state, dtype=dt, device=dev)
    bufs["h"] = torch.empty(B, D, d_state, dtype=torch.float32, device=dev)
    bufs["c"] = torch.empty(B, D, CONV_W - 1, dtype=torch.float32, device=dev)
    bufs["out"] = torch.empty(B, L, DM, dtype=out_dtype or dt, device=dev)
    return bufs


def stages(hidden, weights: dict, params: dict, proj: "_lib.Projector", bufs: dict, stream=None):
    """The layer as a list of (stage name, call), in order; each call enqueues its kernels on
    `stream` and writes into `bufs`."""
    P, b = proj, bufs
    if "xz" in b:
        st = [("in_proj_xz", lambda: P(_lib.PROJ_IN, hidden, weights["in_xz"], out=b["xz"], stream=stream))]
    else:
        st = [("in_proj_x", lambda: P(_lib.PROJ_IN, hidden, weights["in_x"], out=b["x"], stream=stream)),
              ("in_proj_z", lambda: P(_lib.PROJ_IN, hidden, weights["in_z"], out=b["z"], stream=stream))]
    if "u" not in b:
        R = weights["x_dt"].shape[0]
        st.append(("conv_xproj", lambda: _lib.conv_xproj(b["x"], params, weights["x_all"], R, lowrank=b["lowrank"],
                                                         Bm=b["Bm"], Cm=b["Cm"], stream=stream)))
    else:
        st += [("conv_silu", lambda: _lib.conv_silu(b["x"], params, u=b["u"], stream=stream)),
               ("x_proj_dt", lambda: P(_lib.PROJ_X, b["u"], weights["x_dt"], out=b["lowrank"], stream=stream)),
               ("x_proj_B", lambda: P(_lib.PROJ_X, b["u"], weights["x_B"], out=b["Bm"], stream=stream)),
               ("x_proj_C", lambda: P(_lib.PROJ_X, b["u"], weights["x_C"], out=b["Cm"], stream=stream))]
    return st + [
        ("dt_proj", lambda: P(_lib.PROJ_DT, b["lowrank"], weights["dt"], out=b["dt"], stream=stream)),
        ("scan", lambda: _lib.prefill(b["x"], b["dt"], b["z"], b["Bm"], b["Cm"], params, y=b["y"], h_out=b["h"],
                                      conv_out=b["c"], stream=stream)),
        ("out_proj", lambda: P(_lib.PROJ_OUT, b["y"], weights["out"], out=b["out"], stream=stream)),
    ]


def mixer_prefill(hidden, weights: dict, params: dict, proj: "_lib.Projector", *, out_dtype=None, stream=None):
    """Returns (out [B, L, d_model] partial in out_dtype (default: hidden's dtype), h [B, D, N],
    conv [B, D, 3])."""
    bufs = alloc_buffers(hidden, weights, params["A"].shape[1], out_dtype)
    for _, call in stages(hidden, weights, params, proj, bufs, stream):
        call()
    return bufs["out"], bufs["h"], bufs["c"]
