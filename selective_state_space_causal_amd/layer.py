"""One rank's slice of a selective-SSM mixer layer over a prompt, composed from the library's
C-ABI calls (argument marshalling only; every step runs in the library's kernels or in its
hipBLASLt GEMMs):

  x, z    = in_proj (column shard)            [B, L, d_model] -> [B, D, L] each
  u       = conv + SiLU front                 [B, D, L]
  r, B, C = x_proj rows reading these channels [B, D, L] -> [B, L, R], [B, L, N], [B, L, N]
  dt      = dt_proj                           [B, L, R] -> [B, D, L]
  y, h, c = ssm_prefill                       (the scan; leaves the h / conv cache)
  out     = out_proj (row shard)              [B, D, L] -> [B, L, d_model], a partial sum (fp32)

"Scaling State-Space Models on Multiple GPUs with Tensor Parallelism" (euno.news summary of
arXiv 2602.21144), Methodology items 1-2.  With more than one rank, x_proj's outputs and out
are partial sums that the ranks add (all-reduces outside this build); on one GPU the slice's
partials are used as they are.
"""
from __future__ import annotations

import torch

from . import _lib


def mixer_prefill(hidden, weights: dict, params: dict, proj: "_lib.Projector", *, stream=None):
    """Returns (out [B, L, d_model] fp32 partial, h [B, D, N], conv [B, D, 3])."""
    P = proj
    x = P(_lib.PROJ_IN, hidden, weights["in_x"], stream=stream)
    z = P(_lib.PROJ_IN, hidden, weights["in_z"], stream=stream)
    u = _lib.conv_silu(x, params, stream=stream)
    lowrank = P(_lib.PROJ_X, u, weights["x_dt"], stream=stream)
    Bm = P(_lib.PROJ_X, u, weights["x_B"], stream=stream)
    Cm = P(_lib.PROJ_X, u, weights["x_C"], stream=stream)
    dt = P(_lib.PROJ_DT, lowrank, weights["dt"], stream=stream)
    y, h, c = _lib.prefill(x, dt, z, Bm, Cm, params, stream=stream)
    out = P(_lib.PROJ_OUT, y, weights["out"], out_dtype=torch.float32, stream=stream)
    return out, h, c
