"""C ABI of the projections and the conv front (include/ssm_proj.h) without a GPU: exports
and host-side validation.  Every call below is invalid on purpose and must be rejected before
any HIP or hipBLASLt call; the fake context and device addresses are never dereferenced."""
import ctypes
import os
import re

import pytest
import torch

from selective_state_space_causal_amd import _lib as L

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake-pointer tests run only without a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_proj.h")
OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, WORKSPACE = 0, 1, 2, 3, 4, 5, 6
BASE, STEP = 0x7F0000000000, 1 << 32


def fake(i, off=0):
    return ctypes.c_void_p(BASE + i * STEP + off)


def test_exports_every_declared_symbol():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", src)))
    assert names == ["ssm_conv_silu", "ssm_conv_xproj", "ssm_proj", "ssm_proj_create", "ssm_proj_destroy",
                     "ssm_proj_workspace_bytes"]
    lib = L.load()
    for n in names:
        assert hasattr(lib, n)
    assert lib.ssm_proj_workspace_bytes() >= 1 << 20


def proj(kind=L.PROJ_IN, B=1, Ls=64, K=32, M=16, io=L.SSM_BF16, od=L.SSM_BF16, ctx=None, x=None, w=None, out=None,
         ws=None, ws_bytes=None):
    lib = L.load()
    ctx = fake(9) if ctx is None else ctx
    x = fake(0) if x is None else x
    w = fake(1) if w is None else w
    out = fake(2) if out is None else out
    ws = fake(3) if ws is None else ws
    ws_bytes = lib.ssm_proj_workspace_bytes() if ws_bytes is None else ws_bytes
    return lib.ssm_proj(ctx, kind, B, Ls, K, M, io, od, x, w, out, ws, ws_bytes, None)


def test_proj_validation():
    lib = L.load()
    n = ctypes.c_void_p(None)
    assert lib.ssm_proj_create(None) == NULL
    assert proj(ctx=n) == NULL and proj(x=n) == NULL and proj(w=n) == NULL and proj(out=n) == NULL
    for k in (-1, 4, 99):
        assert proj(kind=k) == SHAPE, k
    assert proj(B=0) == SHAPE and proj(Ls=0) == SHAPE and proj(K=0) == SHAPE and proj(M=-1) == SHAPE
    assert proj(B=1 << 40, Ls=1 << 30) == SHAPE          # byte counts overflow
    assert proj(io=2) == DTYPE and proj(od=5) == DTYPE
    assert proj(x=fake(0, 8)) == ALIGN and proj(w=fake(1, 4)) == ALIGN and proj(out=fake(2, 2)) == ALIGN
    assert proj(out=fake(0, 1024)) == ALIAS              # out inside in (64 * 32 * 2 bytes)
    assert proj(out=fake(1, 16)) == ALIAS                # out inside w
    assert proj(ws=n) == WORKSPACE and proj(ws_bytes=1024) == WORKSPACE


def conv(B=2, Ls=64, D=8, io=L.SSM_BF16, dconv=4, x=None, u=None, cw=None, cb=None, c0=None, dims_none=False):
    lib = L.load()
    d = L.Dims(B, Ls, D, 1, dconv, io, 0)
    p = L.Params(None, None, None, (BASE + 5 * STEP) if cw is None else cw, cb)
    x = fake(0) if x is None else x
    u = fake(1) if u is None else u
    return lib.ssm_conv_silu(None if dims_none else ctypes.byref(d), ctypes.byref(p), x, c0, u, None)


def test_conv_validation():
    n = ctypes.c_void_p(None)
    assert conv(dims_none=True) == NULL and conv(x=n) == NULL and conv(u=n) == NULL and conv(cw=0) == NULL
    assert conv(B=0) == SHAPE and conv(Ls=0) == SHAPE and conv(D=0) == SHAPE and conv(dconv=3) == SHAPE
    assert conv(Ls=1 << 31) == SHAPE                     # a row's byte offset must fit 32 bits
    assert conv(io=9) == DTYPE
    assert conv(x=fake(0, 8)) == ALIGN and conv(u=fake(1, 4)) == ALIGN
    assert conv(cw=BASE + 5 * STEP + 8) == ALIGN and conv(cb=BASE + 6 * STEP + 2) == ALIGN
    assert conv(c0=fake(7, 1)) == ALIGN
    assert conv(u=fake(0, 64)) == ALIAS


def xproj(B=2, Ls=64, D=16, N=16, R=8, io=L.SSM_BF16, dconv=4, x=None, w=None, o0=None, o1=None, o2=None,
          cw=None, c0=None, dims_none=False):
    lib = L.load()
    d = L.Dims(B, Ls, D, N, dconv, io, 0)
    p = L.Params(None, None, None, (BASE + 5 * STEP) if cw is None else cw, None)
    x = fake(0) if x is None else x
    w = fake(1) if w is None else w
    o0 = fake(2) if o0 is None else o0
    o1 = fake(3) if o1 is None else o1
    o2 = fake(4) if o2 is None else o2
    return lib.ssm_conv_xproj(None if dims_none else ctypes.byref(d), ctypes.byref(p), x, c0, w, R, o0, o1, o2, None)


def test_conv_xproj_validation():
    n = ctypes.c_void_p(None)
    assert xproj(dims_none=True) == NULL and xproj(x=n) == NULL and xproj(w=n) == NULL and xproj(cw=0) == NULL
    assert xproj(o0=n) == NULL and xproj(o1=n) == NULL and xproj(o2=n) == NULL
    assert xproj(B=0) == SHAPE and xproj(Ls=0) == SHAPE and xproj(D=0) == SHAPE and xproj(R=0) == SHAPE
    assert xproj(N=0) == SHAPE and xproj(N=17) == SHAPE and xproj(dconv=3) == SHAPE
    assert xproj(D=12) == SHAPE and xproj(Ls=60) == SHAPE   # d_inner and seqlen multiples of 8
    assert xproj(B=1 << 40, Ls=1 << 24) == SHAPE           # byte counts overflow
    assert xproj(io=L.SSM_F32) == DTYPE and xproj(io=7) == DTYPE
    assert xproj(x=fake(0, 8)) == ALIGN and xproj(w=fake(1, 4)) == ALIGN and xproj(o1=fake(3, 1)) == ALIGN
    assert xproj(cw=BASE + 5 * STEP + 8) == ALIGN and xproj(c0=fake(7, 2)) == ALIGN
    assert xproj(o0=fake(0, 64)) == ALIAS                  # lowrank inside x
    assert xproj(o2=fake(3, 2)) == ALIAS                   # Cm overlapping Bm
