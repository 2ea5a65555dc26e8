"""One rank's slice of a selective-SSM mixer layer, over a prompt and for one decoded token,
composed from the library's
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
are partial sums that the ranks add (all-reduces that this library does not run); on one GPU the slice's
partials are used as they are.

Decode (mixer_decode_step) runs one token per batch row from the cache the prefill left:
in_proj, then either the four per-token stages as separate calls (conv_silu from the conv
cache, x_proj, dt_proj, ssm_decode_step) or the same four as ssm_decode_fused (two kernels),
then out_proj.

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


# ---- decode: one token per batch row through the layer, from the cache ----

def alloc_decode_buffers(hidden_t, weights: dict, d_state: int, fused: bool, out_dtype=None) -> dict:
    """Every tensor a decode step writes besides the cache, on hidden_t's device."""
    B, DM = hidden_t.shape
    D, R = weights["in_x"].shape[0], weights["x_dt"].shape[0]
    dev, dt = hidden_t.device, hidden_t.dtype
    b = {}
    if B == 1 and "in_xz" in weights:
        b["xz"] = torch.empty(1, 2 * D, 1, dtype=dt, device=dev)
        b["x"], b["z"] = b["xz"][:, :D], b["xz"][:, D:]
    else:
        b["x"] = torch.empty(B, D, 1, dtype=dt, device=dev)
        b["z"] = torch.empty_like(b["x"])
    b["y"] = torch.empty(B, D, 1, dtype=dt, device=dev)
    b["out"] = torch.empty(B, 1, DM, dtype=out_dtype or dt, device=dev)
    if fused:
        b["ws"] = torch.empty(max(1, _lib.decode_fused_workspace_bytes(B, D, R, d_state, dt)), dtype=torch.uint8,
                              device=dev)
        return b
    b["u"] = torch.empty(B, D, 1, dtype=dt, device=dev)
    b["dt"] = torch.empty(B, D, 1, dtype=dt, device=dev)
    if B == 1 and "x_all" in weights:  # one GEMM writes [1, 1, R + 2N]: low-rank, B_t, C_t in a row
        b["xo"] = torch.empty(1, 1, R + 2 * d_state, dtype=dt, device=dev)
        b["lowrank"], b["Bt"], b["Ct"] = (b["xo"][:, :, :R], b["xo"][:, :, R:R + d_state],
                                          b["xo"][:, :, R + d_state:])
    else:
        b["lowrank"] = torch.empty(B, 1, R, dtype=dt, device=dev)
        b["Bt"] = torch.empty(B, 1, d_state, dtype=dt, device=dev)
        b["Ct"] = torch.empty(B, 1, d_state, dtype=dt, device=dev)
    return b


def decode_stages(hidden_t, weights: dict, params: dict, proj: "_lib.Projector", h, conv, bufs: dict,
                  fused: bool, stream=None):
    """One decode step of the layer as a list of (stage name, call); h [B, D, N] and conv
    [B, D, 3] are updated in place.  Unfused: in_proj, conv_silu (from the conv cache), x_proj
    (one GEMM for one batch row with the stacked weight, else three), dt_proj, ssm_decode_step,
    out_proj.  Fused: in_proj, ssm_decode_fused, out_proj."""
    P, b = proj, bufs
    B, DM = hidden_t.shape
    hs = hidden_t.view(B, 1, DM)
    R = weights["x_dt"].shape[0]
    if "xz" in b:
        st = [("in_proj_xz", lambda: P(_lib.PROJ_IN, hs, weights["in_xz"], out=b["xz"], stream=stream))]
    else:
        st = [("in_proj_x", lambda: P(_lib.PROJ_IN, hs, weights["in_x"], out=b["x"], stream=stream)),
              ("in_proj_z", lambda: P(_lib.PROJ_IN, hs, weights["in_z"], out=b["z"], stream=stream))]
    x2, z2, y2 = b["x"].view(B, -1), b["z"].view(B, -1), b["y"].view(B, -1)
    if fused:
        st.append(("decode_fused", lambda: _lib.decode_fused(x2, z2, params, weights["x_all"], weights["dt"], R, h, conv,
                                                             y_t=y2, workspace=b["ws"], stream=stream)))
    else:
        st.append(("conv_silu", lambda: _lib.conv_silu(b["x"], params, conv, u=b["u"], stream=stream)))
        if "xo" in b:
            st.append(("x_proj", lambda: P(_lib.PROJ_X, b["u"], weights["x_all"], out=b["xo"], stream=stream)))
        else:
            st += [("x_proj_dt", lambda: P(_lib.PROJ_X, b["u"], weights["x_dt"], out=b["lowrank"], stream=stream)),
                   ("x_proj_B", lambda: P(_lib.PROJ_X, b["u"], weights["x_B"], out=b["Bt"], stream=stream)),
                   ("x_proj_C", lambda: P(_lib.PROJ_X, b["u"], weights["x_C"], out=b["Ct"], stream=stream))]
        st += [("dt_proj", lambda: P(_lib.PROJ_DT, b["lowrank"], weights["dt"], out=b["dt"], stream=stream)),
               ("decode_step", lambda: _lib.decode_step(x2, b["dt"].view(B, -1), z2, b["Bt"].view(B, -1),
                                                        b["Ct"].view(B, -1), params, h, conv, y_t=y2, stream=stream))]
    st.append(("out_proj", lambda: P(_lib.PROJ_OUT, b["y"], weights["out"], out=b["out"], stream=stream)))
    return st


def mixer_decode_step(hidden_t, weights: dict, params: dict, proj: "_lib.Projector", h, conv, *, fused: bool = True,
                      out_dtype=None, bufs=None, stream=None):
    """One decoded token per batch row: hidden_t [B, d_model]; h [B, D, N] and conv [B, D, 3]
    (the cache) are updated in place.  Returns out [B, d_model], the layer's partial sum.
    fused needs the stacked x_proj weight ("x_all") and d_state 16."""
    if bufs is None:
        bufs = alloc_decode_buffers(hidden_t, weights, params["A"].shape[1], fused, out_dtype)
    for _, call in decode_stages(hidden_t, weights, params, proj, h, conv, bufs, fused, stream):
        call()
    return bufs["out"].view(hidden_t.shape[0], -1)
