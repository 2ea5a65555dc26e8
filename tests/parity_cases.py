"""The cases of the GPU parity tests and the inputs each one runs on.

They live here so that the GPU tests (which compare the HIP path with the oracle) and the CPU
test of the inputs' discriminating power (tests/test_param_discrimination.py, which shows that
the oracle's output moves by many tolerances when a channel's parameters are swapped for
another channel's) build exactly the same seeded inputs.  Every case draws its parameters with
``make_params_distinct``: A, Dskip and conv_b differ from channel to channel, so a kernel that
read another channel's row would fail the comparison.
"""
from __future__ import annotations

import numpy as np
import torch

from selective_state_space_causal_amd import inputs as I

# ---- prefill over awkward shapes: ragged windows, lanes and workgroups ----
EDGE = [
    # B, L, D, N, io, gate, conv_b
    (1, 1, 1, 1, "f32", True, True), (1, 2, 3, 4, "f32", False, True), (2, 3, 5, 16, "bf16", True, False),
    (3, 4, 65, 16, "bf16", True, True), (1, 5, 64, 15, "f32", True, True), (2, 63, 130, 16, "bf16", False, True),
    (1, 64, 7, 8, "f32", True, False), (2, 65, 64, 16, "bf16", True, True), (1, 127, 33, 16, "f32", True, True),
    (1, 513, 3, 16, "bf16", True, True), (1, 1000, 66, 3, "f32", True, True), (3, 777, 129, 16, "bf16", True, True),
]


def edge_inputs(B, L, D, N, io, gate, cb):
    prm = I.make_params_distinct(D, N, seed=L + D)
    if not cb:
        prm["conv_b"] = None
    return prm, I.make_sequence(B, L, D, N, io, seed=B + 7 * L)


# ---- the windowed prefill forced (chunk_hint 8), fresh and resumed from a random cache ----
WINDOWED = [
    # B, L, D, io: aligned and ragged lengths, single-lane and single-window sequences,
    # channel counts that leave idle waves in the last workgroup
    (1, 8, 8, "bf16"), (1, 512, 16, "bf16"), (2, 520, 13, "bf16"), (1, 1024, 9, "f32"), (1, 4104, 24, "bf16"),
    (3, 1536, 17, "f32"), (1, 2000, 8, "bf16"), (2, 7, 3, "f32"), (1, 1030, 31, "bf16"),
]


def windowed_inputs(B, L, D, io):
    return I.make_params_distinct(D, 16, seed=L), I.make_sequence(B, L, D, 16, io, seed=L + 1)


def random_cache(B, D, N, seed, io="f32"):
    """A random cache to resume from: h ~ N(0, 1); the conv window holds raw inputs, so it is
    rounded through the io dtype."""
    g = torch.Generator().manual_seed(seed)
    h0 = torch.randn(B, D, N, generator=g)
    c0 = torch.randn(B, D, 3, generator=g).to(I.io_dtype(io)).float()
    return h0, c0


# ---- decode from a prefilled cache: (io, B, D, N); d_state 16 runs the four-lane kernel,
# others the one-lane kernel; 3 x 130 channels leave a ragged last workgroup ----
DECODE = [("f32", 2, 40, 16), ("bf16", 3, 130, 16), ("bf16", 1, 5, 3)]
DECODE_L, DECODE_T = 97, 24


def decode_inputs(io, B, D, N):
    prm = I.make_params_distinct(D, N, seed=5)
    seq = I.make_sequence(B, DECODE_L, D, N, io, seed=5)
    toks = [I.make_decode_token(B, D, N, t, io, seed=5) for t in range(DECODE_T)]
    return prm, seq, toks


# ---- seeded random sweep: prefill then three decode steps ----
def sweep_cases(n=40, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append(dict(B=int(g.integers(1, 4)), L=int(g.choice([1, 2, 5, 8, 63, 64, 100, 511, 512, 513, 777, 1200])),
                        D=int(g.choice([1, 3, 8, 17, 40, 64, 96])), N=int(g.choice([1, 4, 8, 15, 16, 16, 16])),
                        io=str(g.choice(["f32", "bf16"])), gate=bool(g.integers(0, 2)), resume=bool(g.integers(0, 2)),
                        hint=int(g.choice([0, 0, 1, 8])), seed=1000 + i))
    return out


def sweep_id(c):
    return "B{B}L{L}D{D}N{N}{io}g{gate:d}r{resume:d}h{hint}".format(**c)


def sweep_inputs(c):
    B, L, D, N, io = c["B"], c["L"], c["D"], c["N"], c["io"]
    prm = I.make_params_distinct(D, N, seed=c["seed"])
    seq = I.make_sequence(B, L, D, N, io, seed=c["seed"])
    h0 = c0 = None
    if c["resume"]:
        h0, c0 = random_cache(B, D, N, c["seed"], io)
    toks = [I.make_decode_token(B, D, N, t, io, seed=c["seed"]) for t in range(3)]
    return prm, seq, h0, c0, toks


# ---- the serving form: ragged lengths and cache slots ----
POOL = [(704, 16, "bf16", 0), (701, 16, "bf16", 0), (600, 16, "f32", 0), (300, 8, "bf16", 0), (704, 16, "bf16", 1)]
POOL_B, POOL_D, POOL_S = 5, 40, 7
POOL_LENS = lambda L: [L, 1, 333, 0, L - 5]
POOL_SLOTS = [5, 2, -1, 0, 6]


def pool_inputs(L, N, io):
    return I.make_params_distinct(POOL_D, N, seed=51), I.make_sequence(POOL_B, L, POOL_D, N, io, seed=51)


# ---- the method's degenerate regimes, each on top of per-channel parameters ----
#   a_near_zero  A = -1e-12: exp(delta A) rounds to 1 in fp32, so the state is a running sum;
#   a_huge       A = -1e6: exp(delta A) underflows to 0, so each token's state forgets the past;
#   a_mixed      A[c, n] from -1e-12 to -1e6 over 18 decades, in its own order in every channel;
#   dt_tiny      dt = -60: delta = softplus(...) ~ 1e-28, the step is nearly the identity;
#   dt_huge      dt = +60: delta ~ 55-60, large steps with full decay;
#   x_zero       x = 0: u is the channel's own constant silu(conv_b[c]) at every token.
REGIMES = ["a_near_zero", "a_huge", "a_mixed", "dt_tiny", "dt_huge", "x_zero"]


def regime_params(D, N):
    """Per-channel parameters for the regimes, with the workloads' step range dt0 in [1e-3, 1e-1].
    With steps near 1, the running sums of the regimes whose decay is ~1 (A near zero) grow over
    600 tokens to many times the output they feed, and an output that cancels them holds fp32
    rounding above the fp32 tolerance tau (1 + |y|): 1.1 tau in the one-lane kernel, whose sums
    are one chain of 600 additions, 0.1 tau in the windowed one, whose sums are tree-shaped."""
    return I.make_params_distinct(D, N, seed=17, dt_range=(1e-3, 1e-1))


def regime(name, prm, seq):
    prm, seq = dict(prm), dict(seq)
    D, N = prm["A"].shape
    if name == "a_near_zero":
        prm["A"] = torch.full((D, N), -1e-12, dtype=torch.float32)
    elif name == "a_huge":
        prm["A"] = torch.full((D, N), -1e6, dtype=torch.float32)
    elif name == "a_mixed":
        mags = torch.logspace(-12, 6, N, dtype=torch.float64).to(torch.float32)
        g = torch.Generator().manual_seed(D * 1000 + N)
        prm["A"] = torch.stack([-mags[torch.randperm(N, generator=g)] for _ in range(D)]).contiguous()
    elif name in ("dt_tiny", "dt_huge"):
        seq["dt"] = torch.full_like(seq["dt"], -60.0 if name == "dt_tiny" else 60.0)
    elif name == "x_zero":
        seq["x"] = torch.zeros_like(seq["x"])
    return prm, seq
