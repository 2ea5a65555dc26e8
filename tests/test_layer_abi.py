"""C ABI of the fused per-token layer stages (include/ssm_layer.h) without a GPU: exports, the
workspace query and host-side validation.  Every call below is invalid on purpose and must be
rejected before any HIP call, so the fake device addresses are never used."""
import ctypes
import os
import re

import pytest
import torch

from selective_state_space_causal_amd import _lib as L

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake-pointer tests run only without a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_layer.h")
BASE, STEP = 0x7F0000000000, 1 << 32
NULL, SHAPE, DTYPE, ALIGN, ALIAS, WS, SCRATCH = 1, 2, 3, 4, 5, 6, 8


def fake(i, off=0):
    return ctypes.c_void_p(BASE + i * STEP + off)


def dims(**kw):
    d = dict(batch=2, seqlen=1, d_inner=200, d_state=16, d_conv=4, io_dtype=L.SSM_BF16, chunk_hint=0)
    d.update(kw)
    return L.Dims(**d)


def params(**kw):
    p = dict(A=BASE + 20 * STEP, Dskip=BASE + 21 * STEP, dt_bias=BASE + 22 * STEP, conv_w=BASE + 23 * STEP,
             conv_b=BASE + 24 * STEP)
    p.update(kw)
    return L.Params(**p)


def fused(d, p, rank=24, **over):
    a = dict(wx=fake(0), wdt=fake(1), x=fake(2), z=fake(3), y=fake(4), h=fake(5), conv=fake(6), ws=fake(7),
             ws_bytes=1 << 30)
    a.update(over)
    return L.load().ssm_decode_fused(None if d is None else ctypes.byref(d), None if p is None else ctypes.byref(p),
                                     a["wx"], a["wdt"], rank, a["x"], a["z"], a["y"], a["h"], a["conv"], a["ws"],
                                     a["ws_bytes"], None)


def test_exports_every_declared_symbol():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(ssm_[a-z_]+)\s*\(", src)))
    assert {"ssm_decode_fused", "ssm_decode_fused_workspace_bytes", "ssm_decode_fused_noalloc"} <= set(names)
    lib = L.load()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ssm_layer.h but not exported"


def test_workspace_query():
    lib = L.load()
    # [B, ceil(D / 64), R + 2N] fp32 partial sums
    assert lib.ssm_decode_fused_workspace_bytes(ctypes.byref(dims()), 24) == 2 * 4 * (24 + 32) * 4
    assert lib.ssm_decode_fused_workspace_bytes(ctypes.byref(dims(d_inner=2048, batch=1)), 256) == 32 * 288 * 4
    assert lib.ssm_decode_fused_workspace_bytes(ctypes.byref(dims(d_state=8)), 24) == 0
    assert lib.ssm_decode_fused_workspace_bytes(ctypes.byref(dims()), 481) == 0    # R + 2N > 512
    assert lib.ssm_decode_fused_workspace_bytes(ctypes.byref(dims()), 0) == 0


@pytest.mark.parametrize("kw,rank,code", [
    (dict(batch=0), 24, SHAPE), (dict(d_inner=0), 24, SHAPE), (dict(d_state=8), 24, SHAPE),
    (dict(d_conv=3), 24, SHAPE), (dict(d_inner=(1 << 24) + 1), 24, SHAPE), ({}, 0, SHAPE), ({}, 481, SHAPE),
    (dict(io_dtype=5), 24, DTYPE)])
def test_rejects_bad_sizes(kw, rank, code):
    assert fused(dims(**kw), params(), rank) == code


def test_null_pointers_and_workspace():
    assert fused(None, params()) == NULL
    assert fused(dims(), None) == NULL
    for k in ("wx", "wdt", "x", "y", "h", "conv"):
        assert fused(dims(), params(), **{k: None}) == NULL, k
    assert fused(dims(), params(A=None)) == NULL
    assert fused(dims(), params(), ws=None) == WS
    assert fused(dims(), params(), ws_bytes=2 * 4 * 56 * 4 - 1) == WS


def test_alignment_and_aliasing():
    assert fused(dims(), params(), h=fake(5, 8)) == ALIGN            # h moves as 16-byte vectors
    assert fused(dims(), params(), x=fake(2, 1)) == ALIGN            # bf16 io: 2-byte alignment
    assert fused(dims(), params(A=BASE + 20 * STEP + 4)) == ALIGN
    assert fused(dims(), params(), y=fake(2)) == ALIAS               # y on x
    assert fused(dims(), params(), ws=fake(0)) == ALIAS              # workspace on the weights
    assert fused(dims(), params(), conv=fake(5, 1 << 12)) == ALIAS   # conv inside h


def noalloc(d, p, rank=24, **over):
    a = dict(wx=fake(0), wdt=fake(1), x=fake(2), z=fake(3), y=fake(4), h=fake(5), conv=fake(6))
    a.update(over)
    return L.load().ssm_decode_fused_noalloc(None if d is None else ctypes.byref(d),
                                             None if p is None else ctypes.byref(p), a["wx"], a["wdt"], rank, a["x"],
                                             a["z"], a["y"], a["h"], a["conv"], None)


def test_noalloc_validation_and_scratch_limit():
    """The no-allocation variant validates like ssm_decode_fused and refuses, before any HIP call,
    sizes whose partial sums would not fit its fixed 16 MiB scratch."""
    lib = L.load()
    assert noalloc(None, params()) == NULL
    assert noalloc(dims(), params(), y=None) == NULL
    assert noalloc(dims(d_state=8), params()) == SHAPE
    assert noalloc(dims(), params(), h=fake(5, 8)) == ALIGN
    assert noalloc(dims(), params(), y=fake(2)) == ALIAS
    limit = 16 << 20
    # batch 1024 x 80 blocks of 64 channels x 288 outputs x 4 bytes = 94 MB: too much
    big = dims(batch=1024, d_inner=5120)
    assert lib.ssm_decode_fused_workspace_bytes(ctypes.byref(big), 256) > limit
    assert noalloc(big, params(), rank=256) == SCRATCH
    edge = dims(batch=183, d_inner=5120)   # 183 x 80 x 288 x 4 bytes > 16 MiB; 182 rows fit
    assert lib.ssm_decode_fused_workspace_bytes(ctypes.byref(edge), 256) > limit
    assert noalloc(edge, params(), rank=256) == SCRATCH
    assert lib.ssm_decode_fused_workspace_bytes(ctypes.byref(dims(batch=182, d_inner=5120)), 256) <= limit
    assert lib.ssm_status_str(SCRATCH) != b"unknown status"
