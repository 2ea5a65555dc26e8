"""fp64 CPU oracle for the selective state-space causal scan.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the GPU library: the arithmetic lives in ``ssm_oracle.c`` (plain C, fp64,
libm, one channel at a time, token after token), built here with gcc (or, with
SSM_SANITIZE=1, with clang under AddressSanitizer and UndefinedBehaviorSanitizer).

What it follows: "Scaling State-Space Models on Multiple GPUs with Tensor
Parallelism" (euno.news summary of arXiv 2602.21144), Methodology item 2
(each GPU updates its own channel slice of the hidden state with no
cross-device exchange) and item 3 (prefill leaves the hidden state cached and
decode resumes from it).  The recurrence itself is the standard Mamba
selective-scan form (Gu & Dao, 2023), which the pages do not write out.

Parity pins: none of the pages prints a value of y or h.  This oracle is
pinned instead by brute force, closed forms, limits, library routines and the
pages' two invariants (see ``tests/test_oracle_pins.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
# SSM_SANITIZE=1: a clang build instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
# (the same sanitizer runtime as the library's sanitized build, which the process preloads).
_SANITIZE = os.environ.get("SSM_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "libssm_oracle_san.so" if _SANITIZE else "libssm_oracle.so")
_lib = None

CONV_W = 4


def build(verbose: bool = False) -> str:
    """Compile ssm_oracle.c into oracle/libssm_oracle.so (no fast-math, no FMA contraction);
    with SSM_SANITIZE=1, into oracle/libssm_oracle_san.so with clang and the sanitizers."""
    if _SANITIZE:
        cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fPIC", "-shared", "-std=c99", "-ffp-contract=off",
               "-fno-fast-math", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-shared-libsan",
               "-Wall", "-Wextra", "-o", _LIB, _SRC, "-lm", "-lpthread"]
    else:
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-Wextra", "-o", _LIB, _SRC, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB


def load_library(path: str):
    """Load a compiled oracle (``path``) and declare its entry point."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.ssm_oracle_scan.restype = ctypes.c_int
    lib.ssm_oracle_scan.argtypes = [i64, i64, i64, i64] + [dp] * 15 + [ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = load_library(_LIB)
    return _lib


def _f64(a, shape, name):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: widen exactly on the host
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"oracle: {name} has shape {a.shape}, expected {tuple(shape)}")
    return a


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def scan(x, dt, z, Bm, Cm, A, Dskip, dt_bias, conv_w, conv_b=None,
         h0=None, conv0=None, nthreads: int = 1, lib=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Run the recurrence over all L tokens of every (b, c) channel.

    Shapes: x, dt, z [B, D, L]; Bm, Cm [B, L, N]; A [D, N]; Dskip, dt_bias,
    conv_b [D]; conv_w [D, 4]; h0 [B, D, N]; conv0 [B, D, 3].  ``z``,
    ``conv_b``, ``h0`` and ``conv0`` may be None (no gate, zero bias, zero
    state).  Returns (y [B, D, L], h [B, D, N], conv [B, D, 3]) in fp64.
    """
    x = _f64(x, np.shape(x), "x")
    if x.ndim != 3:
        raise ValueError("oracle: x must be [B, D, L]")
    B, D, L = x.shape
    A = _f64(A, np.shape(A), "A")
    N = A.shape[1]
    dt = _f64(dt, (B, D, L), "dt")
    z = _f64(z, (B, D, L), "z")
    Bm = _f64(Bm, (B, L, N), "Bm")
    Cm = _f64(Cm, (B, L, N), "Cm")
    A = _f64(A, (D, N), "A")
    Dskip = _f64(Dskip, (D,), "Dskip")
    dt_bias = _f64(dt_bias, (D,), "dt_bias")
    conv_w = _f64(conv_w, (D, CONV_W), "conv_w")
    conv_b = _f64(conv_b, (D,), "conv_b")
    h0 = _f64(h0, (B, D, N), "h0")
    conv0 = _f64(conv0, (B, D, CONV_W - 1), "conv0")
    y = np.empty((B, D, L), np.float64)
    h = np.empty((B, D, N), np.float64)
    conv = np.empty((B, D, CONV_W - 1), np.float64)
    rc = (lib or _load()).ssm_oracle_scan(B, L, D, N, _ptr(x), _ptr(dt), _ptr(z), _ptr(Bm), _ptr(Cm),
                                 _ptr(A), _ptr(Dskip), _ptr(dt_bias), _ptr(conv_w), _ptr(conv_b),
                                 _ptr(h0), _ptr(conv0), _ptr(y), _ptr(h), _ptr(conv), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle: ssm_oracle_scan failed")
    return y, h, conv


def prefill(seq: dict, params: dict, nthreads: int = 1, gate: bool = True):
    """Fresh prefill (zero state, zero conv history) of one sequence batch."""
    return scan(seq["x"], seq["dt"], seq["z"] if gate else None, seq["Bm"], seq["Cm"],
                params["A"], params["Dskip"], params["dt_bias"], params["conv_w"],
                params.get("conv_b"), nthreads=nthreads)


def decode_step(tok: dict, params: dict, h, conv, gate: bool = True, nthreads: int = 1):
    """One decode step from the cache (h [B,D,N], conv [B,D,3]).

    ``tok`` holds x, dt, z as [B, D] and Bm, Cm as [B, N].  Returns
    (y [B, D], h_new, conv_new); the inputs are not modified.
    """
    x = np.asarray(_f64(tok["x"], np.shape(tok["x"]), "x"))[..., None]
    Bsz, D = x.shape[:2]
    y, h2, c2 = scan(x, _f64(tok["dt"], (Bsz, D), "dt")[..., None],
                     _f64(tok["z"], (Bsz, D), "z")[..., None] if gate else None,
                     _f64(tok["Bm"], np.shape(tok["Bm"]), "Bm")[:, None, :],
                     _f64(tok["Cm"], np.shape(tok["Cm"]), "Cm")[:, None, :],
                     params["A"], params["Dskip"], params["dt_bias"], params["conv_w"],
                     params.get("conv_b"), h0=h, conv0=conv, nthreads=nthreads)
    return y[..., 0], h2, c2


def scan_channels(seq: dict, params: dict, pairs: Iterable[Tuple[int, int]],
                  gate: bool = True, h0=None, conv0=None):
    """Oracle for a sample of (b, c) channels only (the recurrence is channel-local).

    ``seq`` tensors may be torch tensors on any device or numpy arrays; only
    the sampled rows are copied to the host.  Returns a list of
    (y [L], h [N], conv [3]) per pair, fp64.
    """
    out = []
    for b, c in pairs:
        def row(t):
            r = t[b:b + 1, c:c + 1]
            return r
        sl = slice(c, c + 1)
        y, h, conv = scan(row(seq["x"]), row(seq["dt"]), row(seq["z"]) if gate else None,
                          seq["Bm"][b:b + 1], seq["Cm"][b:b + 1],
                          params["A"][sl], params["Dskip"][sl], params["dt_bias"][sl],
                          params["conv_w"][sl],
                          None if params.get("conv_b") is None else params["conv_b"][sl],
                          h0=None if h0 is None else h0[b:b + 1, c:c + 1],
                          conv0=None if conv0 is None else conv0[b:b + 1, c:c + 1])
        out.append((y[0, 0], h[0, 0], conv[0, 0]))
    return out
