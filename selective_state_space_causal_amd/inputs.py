"""Seeded synthetic inputs for the selective-SSM scan (shared by the GPU path's
tests/bench and the oracle; holds none of the scan's arithmetic).

Recipe (the pages measure on trained Mamba / Falcon-Mamba / Zamba layers over
2K-64K contexts -- "Scaling State-Space Models on Multiple GPUs with Tensor
Parallelism", Methodology item 5 -- these synthetic layers stand in for them):
  x, z, B, C ~ N(0, 1)                 dt (raw step) ~ N(0, 0.5^2)
  per channel: dt0 log-uniform in [lo, hi], dt_bias = log(expm1(dt0))
  A[c, n] = -exp(A_log[n]), A_log[n] = log(n + 1)
  Dskip = 1, conv_w ~ U(-0.5, 0.5), conv_b = 0
  B and C are shared by all channels of a batch row (per token, per state).
io tensors are drawn in fp32 and rounded to bf16 (round-to-nearest-even) when
io is bf16; parameters are fp32.  Every tensor has its own stream, keyed by
(seed, tensor name, step), so a decode token's inputs do not depend on L.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

CONV_W = 4


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    d_inner: int
    d_state: int
    io: str                      # "f32" or "bf16"
    dt_range: Tuple[float, float] = (1e-3, 1e-1)
    decode_steps: int = 0
    note: str = ""


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 16, 4, "f32", note="tiny fp32 case the oracle runs in milliseconds"),
    "mamba130m": Workload("mamba130m", 4, 2048, 1536, 16, "bf16", note="Mamba-130M-shaped layer, prefill"),
    "mamba2.8b": Workload("mamba2.8b", 64, 8192, 5120, 16, "bf16", decode_steps=256,
                          note="Mamba-2.8B-shaped layer, prefill then 256 decode steps"),
    "slice7b": Workload("slice7b", 1, 32768, 2048, 16, "bf16", decode_steps=128,
                        note="7B-class channel slice (2048 of 8192 channels), prefill then 128 decode steps"),
    "long64k": Workload("long64k", 2, 65536, 7424, 16, "bf16", dt_range=(1e-4, 1e-1),
                        note="long context, prefill only"),
}


def io_dtype(io: str) -> torch.dtype:
    if io == "f32":
        return torch.float32
    if io == "bf16":
        return torch.bfloat16
    raise ValueError(f"unknown io dtype {io!r}")


def _key(k) -> int:
    return zlib.crc32(k.encode()) if isinstance(k, str) else int(k)


def rng(seed: int, *keys) -> np.random.Generator:
    """Independent PCG64 stream for (seed, *keys)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed)] + [_key(k) for k in keys])))


def torch_seed(seed: int, *keys) -> int:
    ss = np.random.SeedSequence([int(seed)] + [_key(k) for k in keys])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(2**63 - 1))


def make_params(d_inner: int, d_state: int, seed: int = 0,
                dt_range: Tuple[float, float] = (1e-3, 1e-1)) -> dict:
    """Per-channel parameters, fp32 torch tensors on the host."""
    D, N = d_inner, d_state
    lo, hi = dt_range
    g = rng(seed, "dt0")
    dt0 = np.exp(g.uniform(np.log(lo), np.log(hi), size=D))
    dt_bias = np.log(np.expm1(dt0))
    A_log = np.log(np.arange(1, N + 1, dtype=np.float64))
    A = np.broadcast_to(-np.exp(A_log), (D, N))
    conv_w = rng(seed, "conv_w").uniform(-0.5, 0.5, size=(D, CONV_W))
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return {"A": f(A), "Dskip": f(np.ones(D)), "dt_bias": f(dt_bias),
            "conv_w": f(conv_w), "conv_b": f(np.zeros(D))}


def _separated(g: np.random.Generator, n: int, lo: float, hi: float) -> np.ndarray:
    """n values in [lo, hi], each at least 0.6 (hi - lo) / 5 away from the previous channel's
    value and from channel 0's: [lo, hi] is cut into five bins, channel 0 takes a random bin,
    every other channel one of the four remaining bins, never its predecessor's, and each value
    lies in the middle 40% of its bin."""
    w = (hi - lo) / 5.0
    bins = np.empty(n, dtype=np.int64)
    bins[0] = g.integers(5)
    if n > 1:
        others = np.array([k for k in range(5) if k != bins[0]])
        walk = (g.integers(4) + np.cumsum(g.integers(1, 4, size=n - 1))) % 4
        bins[1:] = others[walk]
    return lo + w * (bins + g.uniform(0.3, 0.7, size=n))


def make_params_distinct(d_inner: int, d_state: int, seed: int = 0,
                         dt_range: Tuple[float, float] = (1e-2, 1.0)) -> dict:
    """Per-channel parameters for parity tests, every channel's rows drawn on their own, so
    that reading another channel's parameters changes the result:
      A[c, n] = -10^U(-2, 2), independent per (channel, state): magnitudes over four decades
              in no order along n or c;
      Dskip[c] in [0.25, 2], conv_b[c] in [-0.6, 0.6], each well apart from the previous
              channel's value and from channel 0's (_separated);
      dt_bias and conv_w as in make_params (already per channel), with steps dt0 in
              [1e-2, 1] so that the state, and with it A, weighs in the output at bf16
              tolerance.
    The workloads' own distributions (make_params) give every channel the same A row, unit
    D-skip and zero conv bias; those stay the benchmark's inputs."""
    p = make_params(d_inner, d_state, seed=seed, dt_range=dt_range)
    D, N = d_inner, d_state
    g = rng(seed, "distinct")
    A = -np.power(10.0, g.uniform(-2.0, 2.0, size=(D, N)))
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    p["A"] = f(A)
    p["Dskip"] = f(_separated(g, D, 0.25, 2.0))
    p["conv_b"] = f(_separated(g, D, -0.6, 0.6))
    return p


def make_sequence(batch: int, seqlen: int, d_inner: int, d_state: int, io: str = "bf16",
                  seed: int = 0, stream="prefill", dt_std: float = 0.5) -> dict:
    """x, dt, z [B, D, L] and Bm, Cm [B, L, N] as host torch tensors of the io dtype."""
    Bsz, L, D, N = batch, seqlen, d_inner, d_state
    dtype = io_dtype(io)

    def normal(name, shape, scale=1.0):
        a = rng(seed, stream, name).standard_normal(size=shape, dtype=np.float32)
        if scale != 1.0:
            a *= np.float32(scale)
        return torch.from_numpy(a).to(dtype)

    return {"x": normal("x", (Bsz, D, L)), "dt": normal("dt", (Bsz, D, L), dt_std),
            "z": normal("z", (Bsz, D, L)), "Bm": normal("B", (Bsz, L, N)),
            "Cm": normal("C", (Bsz, L, N))}


def make_sequence_device(batch: int, seqlen: int, d_inner: int, d_state: int, io: str = "bf16",
                         seed: int = 0, stream="prefill", device="cuda", dt_std: float = 0.5) -> dict:
    """Same recipe generated with torch's device RNG, for sizes too large to draw on the host.

    The values differ from ``make_sequence`` (another generator) but have the
    same distributions; they are seeded and reproducible on one torch build.
    """
    Bsz, L, D, N = batch, seqlen, d_inner, d_state
    dtype = io_dtype(io)

    def normal(name, shape, scale=1.0):
        g = torch.Generator(device=device)
        g.manual_seed(torch_seed(seed, stream, name))
        out = torch.empty(shape, dtype=dtype, device=device)
        # draw in chunks of whole batch rows, up to 2^26 values, to bound the fp32 temporary
        flat = out.view(shape[0], -1)
        rows = max(1, (1 << 26) // max(1, flat.shape[1]))
        for r0 in range(0, shape[0], rows):
            r1 = min(shape[0], r0 + rows)
            t = torch.randn(r1 - r0, flat.shape[1], generator=g, device=device, dtype=torch.float32)
            if scale != 1.0:
                t.mul_(scale)
            flat[r0:r1].copy_(t)
            del t
        return out

    return {"x": normal("x", (Bsz, D, L)), "dt": normal("dt", (Bsz, D, L), dt_std),
            "z": normal("z", (Bsz, D, L)), "Bm": normal("B", (Bsz, L, N)),
            "Cm": normal("C", (Bsz, L, N))}


def make_decode_token(batch: int, d_inner: int, d_state: int, step: int, io: str = "bf16",
                      seed: int = 0) -> dict:
    """Inputs of decode step ``step``: x, dt, z [B, D]; Bm, Cm [B, N]."""
    s = make_sequence(batch, 1, d_inner, d_state, io, seed, stream=f"decode{step}")
    return {"x": s["x"][..., 0].contiguous(), "dt": s["dt"][..., 0].contiguous(),
            "z": s["z"][..., 0].contiguous(), "Bm": s["Bm"][:, 0].contiguous(),
            "Cm": s["Cm"][:, 0].contiguous()}


# ---- the tensor-parallel aggregation tensor (input of the int8 codec) ----
#
# Under tensor parallelism each rank's slice of the mixer ends in a partial output
# [tokens, d_model] that the ranks sum (page 1, Methodology item 4).  Stand-in recipe:
# every element N(0, 1) times a per-token magnitude log-uniform in [1e-2, 1e2], so blocks
# along d_model see scales that differ by orders of magnitude from token to token.  Each
# rank's part has its own stream.

@dataclass(frozen=True)
class AggregateWorkload:
    name: str
    tokens: int
    d_model: int
    parts: int                   # tensor-parallel ranks whose parts are summed
    block: int                   # elements per int8 scale
    io: str
    note: str = ""


AGGREGATES = {
    "tp_prefill_7b": AggregateWorkload("tp_prefill_7b", 32768, 4096, 4, 128, "bf16",
                                       note="7B-class layer (d_model 4096), 32K-token prefill, 4 ranks"),
    "tp_decode_2.8b": AggregateWorkload("tp_decode_2.8b", 64, 2560, 4, 128, "bf16",
                                        note="Mamba-2.8B-shaped layer (d_model 2560), one decode token for "
                                             "a batch of 64, 4 ranks"),
}


def make_aggregate(tokens: int, d_model: int, io: str = "bf16", seed: int = 0, part: int = 0,
                   device="cpu") -> torch.Tensor:
    """One rank's partial output [tokens, d_model] (recipe above), drawn with torch's RNG on
    `device` (values depend on the device's generator; seeded and reproducible)."""
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, "aggregate", part))
    mag = torch.exp(torch.empty(tokens, 1, device=device).uniform_(float(np.log(1e-2)), float(np.log(1e2)),
                                                                    generator=g))
    out = torch.empty(tokens, d_model, dtype=io_dtype(io), device=device)
    rows = max(1, (1 << 24) // d_model)  # bound the fp32 temporary
    for r0 in range(0, tokens, rows):
        r1 = min(tokens, r0 + rows)
        t = torch.randn(r1 - r0, d_model, generator=g, device=device, dtype=torch.float32)
        out[r0:r1].copy_(t.mul_(mag[r0:r1]))
        del t
    return out


# ---- the channel-sliced projections around the scan (one rank's shard of a mixer layer) ----
#
# Page 1 (Methodology item 1) splits the mixer's projection weights across GPUs along the
# feature dimension.  Stand-in weights for one rank's shard, random-initialised at the usual
# 1/sqrt(fan_in) scale (no trained weights are used):
#   in_xz [2D, d_model]          N(0, 1/d_model)   column shard of the input projection: rows
#                                                  [0, D) make x (in_x), rows [D, 2D) make z (in_z)
#   x_all [R + 2N, D]            N(0, 1/D)         the rows of x_proj that read these channels:
#                                                  x_dt [R, D], then x_B [N, D], then x_C [N, D]
#   dt [D, R]                    N(0, 1/R) * 0.5   step-size projection of these channels
#   out [d_model, D]             N(0, 1/D)         row shard of the output projection
# and the layer input hidden [B, L, d_model] ~ N(0, 1).  io tensors are rounded to bf16 (RNE).

@dataclass(frozen=True)
class LayerWorkload:
    name: str
    batch: int
    seqlen: int
    d_model: int
    d_inner: int                 # this rank's channels
    dt_rank: int
    d_state: int
    io: str
    note: str = ""


LAYERS = {
    "layer7b": LayerWorkload("layer7b", 1, 32768, 4096, 2048, 256, 16, "bf16",
                             note="7B-class mixer layer (d_model 4096, d_inner 8192 split 4 ways), 32K-token "
                                  "prefill: this rank's projections, conv front, scan"),
    "layer_small": LayerWorkload("layer_small", 2, 200, 96, 64, 8, 16, "bf16",
                                 note="small layer the oracle runs in seconds"),
}


def make_proj_weights(d_model: int, d_inner: int, dt_rank: int, d_state: int, io: str = "bf16", seed: int = 0,
                      device="cpu") -> dict:
    dtype = io_dtype(io)

    def normal(name, shape, std):
        g = torch.Generator(device=device)
        g.manual_seed(torch_seed(seed, "proj", name))
        return (torch.randn(shape, generator=g, device=device) * std).to(dtype)

    # in_proj's shard is one [2 d_inner, d_model] tensor (x rows, then z rows); in_x and in_z
    # are its halves (views).
    in_xz = torch.cat([normal("in_x", (d_inner, d_model), d_model ** -0.5),
                       normal("in_z", (d_inner, d_model), d_model ** -0.5)])
    # x_proj's rows that read these channels, stacked likewise: low-rank, then B, then C.
    x_all = torch.cat([normal("x_dt", (dt_rank, d_inner), d_inner ** -0.5),
                       normal("x_B", (d_state, d_inner), d_inner ** -0.5),
                       normal("x_C", (d_state, d_inner), d_inner ** -0.5)])
    return {"in_xz": in_xz, "in_x": in_xz[:d_inner], "in_z": in_xz[d_inner:],
            "x_all": x_all, "x_dt": x_all[:dt_rank], "x_B": x_all[dt_rank:dt_rank + d_state],
            "x_C": x_all[dt_rank + d_state:],
            "dt": normal("dt", (d_inner, dt_rank), 0.5 * dt_rank ** -0.5),
            "out": normal("out", (d_model, d_inner), d_inner ** -0.5)}


def make_hidden(batch: int, seqlen: int, d_model: int, io: str = "bf16", seed: int = 0, device="cpu") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, "hidden"))
    out = torch.empty(batch, seqlen, d_model, dtype=io_dtype(io), device=device)
    for b in range(batch):
        out[b].copy_(torch.randn(seqlen, d_model, generator=g, device=device))
    return out
