"""Helpers for the GPU parity tests (oracle on the host, HIP path on the device)."""
from __future__ import annotations

import os
import re

import numpy as np
import torch

import oracle
from selective_state_space_causal_amd import inputs as I

TAU = {"f32": 1e-4, "bf16": 2e-2}   # |gpu - ref| <= tau * (1 + |ref|), elementwise
DEV = "cuda:0"


def threads():
    return max(1, min(16, oracle.default_threads()))


def dev(d):
    return {k: (None if v is None else v.to(DEV)) for k, v in d.items()}


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


# Observed parity margins: for every test, the largest |gpu - ref| / (1 + |ref|) seen per
# output kind ("y" or "h"), with the tolerance it was held to, and for the full-size decode
# runs one value per step.  conftest.py writes them to the JSON file named by
# SSM_PARITY_MARGINS at the end of the session.
MARGINS = {}


def _test_id():
    return os.environ.get("PYTEST_CURRENT_TEST", "?").rsplit(" (", 1)[0]


def _kind(what):
    m = re.search(r"(?:^|\s)(y|h)(?=\s|\[|$)", what)
    return m.group(1) if m else "other"


def record_margin(err, tau, kind, step=None, tight=None):
    rec = MARGINS.setdefault(_test_id(), {})
    k = rec.setdefault(kind, {"err": 0.0, "tau": tau})
    k["err"] = max(k["err"], float(err))
    if tight is not None:
        k["tight"] = max(k.get("tight", 0.0), float(tight))
    if step is not None:
        series = rec.setdefault("per_step", {}).setdefault(kind, [])
        while len(series) <= step:
            series.append(0.0)
        series[step] = max(series[step], float(err))


FP32_TAU = 1e-4


def tight_ratio(gpu, ref, tau, kind):
    """How much of a tighter bar than tau the error uses, for bf16 io (tau 2e-2, about five
    times the output's own rounding).  The arithmetic runs in fp32 on exactly widened inputs, so
    h is held to the fp32 bar 1e-4 (1 + |ref|), and y to the rounding of the bf16 output (at
    most half an ulp, 2^-8 |y|) plus twice the fp32 bar.  assert_close requires the ratio to stay
    at or below 1, so that an accuracy regression of the fp32 arithmetic cannot hide under the
    bf16 tolerance.  Returns max(|gpu - ref| / bar), or None where no such bar applies."""
    if tau != TAU["bf16"] or kind not in ("y", "h"):
        return None
    a = np.abs(ref)
    bar = (2.0 ** -8 * a + 2 * FP32_TAU * (1.0 + a)) if kind == "y" else FP32_TAU * (1.0 + a)
    return float((np.abs(gpu - ref) / bar).max())


def assert_close(gpu, ref, tau, what, step=None, exact_inputs=True):
    """|gpu - ref| <= tau (1 + |ref|) elementwise, recorded in MARGINS.  exact_inputs: the GPU
    and the oracle start from the same io bits, so the tight bf16 bar (tight_ratio) applies too;
    False where intermediates the two sides round independently (a layer's projections) feed
    the compared values."""
    gpu = f64(gpu) if torch.is_tensor(gpu) else np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if gpu.size == 0:
        return 0.0
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref) / (1.0 + np.abs(ref))
    i = np.unravel_index(err.argmax(), err.shape)
    kind = _kind(what)
    tight = tight_ratio(gpu, ref, tau, kind) if exact_inputs else None
    record_margin(err.max(), tau, kind, step, tight)
    assert err.max() <= tau, f"{what}: max err {err.max():.3e} > {tau:.0e} at {i}: gpu {gpu[i]!r} ref {ref[i]!r}"
    assert tight is None or tight <= 1.0, f"{what}: error {tight:.3f} x the fp32 bar (bf16 rounding aside)"
    return float(err.max())


def assert_bitwise(gpu, ref, what):
    gpu = f64(gpu) if torch.is_tensor(gpu) else np.asarray(gpu, np.float64)
    assert np.array_equal(gpu, np.asarray(ref, np.float64)), f"{what}: not bit-exact"


def note(msg):
    print(msg, flush=True)


def sample_pairs(B, D, k, seed=0):
    g = np.random.default_rng(seed)
    fixed = {(0, 0), (B - 1, D - 1), (0, D - 1), (B - 1, 0), (0, min(63, D - 1)), (B - 1, min(64, D - 1))}
    rnd = {(int(g.integers(B)), int(g.integers(D))) for _ in range(k)}
    return sorted(fixed | rnd)
