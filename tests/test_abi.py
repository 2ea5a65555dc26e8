"""C ABI of libssm.so without a GPU: exports and host-side validation.

Every call below is invalid on purpose and must be rejected before any HIP call, so the
fake device addresses are never dereferenced or launched on."""
import ctypes
import os
import re

import pytest
import torch

from selective_state_space_causal_amd import _lib as L

# The fake device addresses below must never reach a kernel.  Validation rejects every one of
# these calls first; still, where a GPU is visible a validation bug would fault it, so there
# the same error paths are exercised with real tensors by the GPU tests instead.
# (device_count() does not initialise the HIP runtime.)
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake-pointer tests run only without a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = L.load()
    names = declared_functions()
    assert {"ssm_prefill", "ssm_decode_step", "ssm_prefill_workspace_bytes", "ssm_abi_version",
            "ssm_status_str"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ssm.h but not exported"


def test_version_and_status_strings():
    lib = L.load()
    assert lib.ssm_abi_version() == L.ABI_VERSION
    for code in range(9):
        assert lib.ssm_status_str(code) != b"unknown status", code
    assert lib.ssm_status_str(99) == b"unknown status"


BASE = 0x7F0000000000
STEP = 1 << 32  # far apart: no accidental overlaps


def fake(i, off=0):
    return ctypes.c_void_p(BASE + i * STEP + off)


def dims(**kw):
    d = dict(batch=2, seqlen=64, d_inner=32, d_state=16, d_conv=4, io_dtype=L.SSM_BF16, chunk_hint=0)
    d.update(kw)
    return L.Dims(**d)


def params(**kw):
    p = dict(A=BASE + 20 * STEP, Dskip=BASE + 21 * STEP, dt_bias=BASE + 22 * STEP, conv_w=BASE + 23 * STEP,
             conv_b=BASE + 24 * STEP)
    p.update(kw)
    return L.Params(**p)


def prefill(d, p, **over):
    a = dict(x=fake(0), dt=fake(1), z=fake(2), Bm=fake(3), Cm=fake(4), h0=None, conv0=None, y=fake(5),
             h_out=fake(6), conv_out=fake(7), ws=None, ws_bytes=0)
    a.update(over)
    lib = L.load()
    return lib.ssm_prefill(None if d is None else ctypes.byref(d), None if p is None else ctypes.byref(p),
                           a["x"], a["dt"], a["z"], a["Bm"], a["Cm"], a["h0"], a["conv0"], a["y"],
                           a["h_out"], a["conv_out"], a["ws"], a["ws_bytes"], None)


def decode(d, p, **over):
    a = dict(x=fake(0), dt=fake(1), z=fake(2), Bt=fake(3), Ct=fake(4), y=fake(5), h=fake(6), conv=fake(7))
    a.update(over)
    return L.load().ssm_decode_step(None if d is None else ctypes.byref(d), None if p is None else ctypes.byref(p),
                                    a["x"], a["dt"], a["z"], a["Bt"], a["Ct"], a["y"], a["h"], a["conv"], None)


NULL, SHAPE, DTYPE, ALIGN, ALIAS, WS = 1, 2, 3, 4, 5, 6


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), SHAPE), (dict(seqlen=0), SHAPE), (dict(d_inner=-1), SHAPE), (dict(d_state=0), SHAPE),
    (dict(d_state=17), SHAPE), (dict(d_conv=3), SHAPE), (dict(chunk_hint=-2), SHAPE), (dict(chunk_hint=3), SHAPE),
    (dict(batch=1 << 40, d_inner=1 << 20), SHAPE), (dict(d_inner=(1 << 24) + 1), SHAPE),
    (dict(batch=1 << 20, seqlen=1 << 40), SHAPE), (dict(io_dtype=7), DTYPE)])
def test_prefill_rejects_bad_dims(kw, code):
    assert prefill(dims(**kw), params()) == code


def test_prefill_null_pointers():
    assert prefill(None, params()) == NULL
    assert prefill(dims(), None) == NULL
    for k in ("x", "dt", "Bm", "Cm", "y", "h_out", "conv_out"):
        assert prefill(dims(), params(), **{k: None}) == NULL, k
    for k in ("A", "Dskip", "dt_bias", "conv_w"):
        assert prefill(dims(), params(**{k: None})) == NULL, k


def test_prefill_alignment():
    for k in ("x", "dt", "z", "Bm", "Cm", "y", "h_out", "conv_out"):
        assert prefill(dims(), params(), **{k: fake(0 if k != "x" else 9, 8)}) == ALIGN, k
    assert prefill(dims(), params(), h0=fake(10, 4)) == ALIGN
    assert prefill(dims(), params(conv_b=BASE + 24 * STEP + 2)) == ALIGN
    assert prefill(dims(), params(A=BASE + 20 * STEP + 4)) == ALIGN
    assert prefill(dims(), params(conv_w=BASE + 23 * STEP + 8)) == ALIGN


def test_prefill_aliasing():
    seq_bytes = 2 * 32 * 64 * 2
    assert prefill(dims(), params(), y=fake(0, 16)) == ALIAS                      # y inside x
    assert prefill(dims(), params(), y=fake(0, seq_bytes - 16)) == ALIAS          # y's head on x's tail
    assert prefill(dims(), params(), h_out=fake(7, 0)) == ALIAS                   # h_out == conv_out
    assert prefill(dims(), params(), conv_out=fake(3, 0)) == ALIAS                # conv_out over Bm
    assert prefill(dims(), params(), h_out=ctypes.c_void_p(BASE + 20 * STEP)) == ALIAS   # over A
    assert prefill(dims(), params(), h0=fake(6, 0)) == ALIAS                      # h_out over h0
    assert prefill(dims(), params(), conv0=fake(7, 0)) == ALIAS                   # conv_out over conv0


def test_decode_validation():
    assert decode(None, params()) == NULL
    assert decode(dims(seqlen=0), params(), x=None) == NULL        # seqlen is ignored by decode
    assert decode(dims(d_state=20), params()) == SHAPE
    assert decode(dims(io_dtype=4), params()) == DTYPE
    for k in ("x", "dt", "Bt", "Ct", "y", "h", "conv"):
        assert decode(dims(), params(), **{k: None}) == NULL, k
    assert decode(dims(), params(), h=fake(6, 4)) == ALIGN
    assert decode(dims(), params(), x=fake(0, 1)) == ALIGN            # bf16 needs 2-byte alignment
    assert decode(dims(), params(), conv=fake(7, 2)) == ALIGN
    assert decode(dims(io_dtype=L.SSM_F32), params(), y=fake(5, 2)) == ALIGN
    assert decode(dims(), params(), y=fake(0)) == ALIAS            # y_t over x_t
    assert decode(dims(), params(), conv=fake(6, 256)) == ALIAS    # conv inside h
    assert decode(dims(), params(), h=ctypes.c_void_p(BASE + 23 * STEP)) == ALIAS   # h over conv_w


def test_workspace_query_is_host_only():
    lib = L.load()
    for kw in (dict(), dict(batch=64, seqlen=8192, d_inner=5120), dict(batch=1, seqlen=32768, d_inner=2048)):
        d = dims(**kw)
        assert lib.ssm_prefill_workspace_bytes(ctypes.byref(d)) >= 0
    assert lib.ssm_prefill_workspace_bytes(ctypes.byref(dims(batch=0))) == 0
    assert lib.ssm_prefill_workspace_bytes(None) == 0


def test_binding_fails_loudly_without_library(tmp_path):
    saved = L._lib
    L._lib = None
    try:
        with pytest.raises(ImportError):
            L.load(str(tmp_path / "missing.so"))
    finally:
        L._lib = saved


def prefill_pool(d, p, **over):
    a = dict(x=fake(0), dt=fake(1), z=fake(2), Bm=fake(3), Cm=fake(4), seqlens=fake(8), slots=fake(9), pool=6,
             resume=0, y=fake(5), h=fake(6), conv=fake(7))
    a.update(over)
    return L.load().ssm_prefill_pool(None if d is None else ctypes.byref(d), None if p is None else ctypes.byref(p),
                                     a["x"], a["dt"], a["z"], a["Bm"], a["Cm"], a["seqlens"], a["slots"], a["pool"],
                                     a["resume"], a["y"], a["h"], a["conv"], None)


def decode_pool(d, p, **over):
    a = dict(x=fake(0), dt=fake(1), z=fake(2), Bt=fake(3), Ct=fake(4), slots=fake(9), pool=6, y=fake(5), h=fake(6),
             conv=fake(7))
    a.update(over)
    return L.load().ssm_decode_step_pool(None if d is None else ctypes.byref(d), None if p is None else ctypes.byref(p),
                                         a["x"], a["dt"], a["z"], a["Bt"], a["Ct"], a["slots"], a["pool"], a["y"],
                                         a["h"], a["conv"], None)


def test_pool_entry_points_validation():
    for fn in (prefill_pool, decode_pool):
        assert fn(None, params()) == NULL
        assert fn(dims(), params(), slots=None) == NULL
        assert fn(dims(), params(), h=None) == NULL
        assert fn(dims(), params(), pool=0) == SHAPE
        assert fn(dims(), params(), pool=1 << 60) == SHAPE   # S * D * N * 4 bytes overflow
        assert fn(dims(d_state=0), params()) == SHAPE
        assert fn(dims(), params(), slots=fake(9, 2)) == ALIGN
        assert fn(dims(), params(), h=fake(6, 4)) == ALIGN
        assert fn(dims(), params(), h=fake(0)) == ALIAS            # pool over x
        assert fn(dims(), params(), slots=fake(5)) == ALIAS        # y over slots
        assert fn(dims(), params(), conv=fake(6, 64)) == ALIAS     # conv pool inside the h pool
    assert prefill_pool(dims(), params(), seqlens=fake(8, 2)) == ALIGN
    assert prefill_pool(dims(), params(), seqlens=fake(5, 0)) == ALIAS   # y over seqlens
    assert prefill_pool(dims(chunk_hint=5), params()) == SHAPE


def test_binding_refuses_host_tensors():
    """Tensors in host memory are refused by the binding before any HIP call (the kernels would
    read them as device addresses)."""
    import torch

    import selective_state_space_causal_amd as ssm
    from selective_state_space_causal_amd import inputs as I

    B, L, D, N = 1, 16, 8, 16
    prm = I.make_params(D, N)
    s = I.make_sequence(B, L, D, N, "bf16")
    with pytest.raises(ValueError, match="GPU"):
        ssm.prefill(s["x"], s["dt"], s["z"], s["Bm"], s["Cm"], prm)
    tok = I.make_decode_token(B, D, N, 0, "bf16")
    h, c = torch.zeros(B, D, N), torch.zeros(B, D, 3)
    with pytest.raises(ValueError, match="GPU"):
        ssm.decode_step(tok["x"], tok["dt"], tok["z"], tok["Bm"], tok["Cm"], prm, h, c)
