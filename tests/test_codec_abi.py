"""C ABI of the block int8 codec (include/ssm_codec.h) without a GPU: exports and host-side
validation.  Every call below is invalid on purpose and must be rejected before any HIP call,
so the fake device addresses are never dereferenced or launched on."""
import ctypes
import os
import re

import pytest
import torch

from selective_state_space_causal_amd import _lib as L

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake-pointer tests run only without a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_codec.h")

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS = 0, 1, 2, 3, 4, 5
BASE = 0x7F0000000000
STEP = 1 << 32


def fake(i, off=0):
    return ctypes.c_void_p(BASE + i * STEP + off)


def test_exports_every_declared_symbol():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", src)))
    assert names == ["ssm_q8_dequant_sum", "ssm_q8_num_blocks", "ssm_q8_quantize"]
    lib = L.load()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ssm_codec.h but not exported"


def test_num_blocks():
    lib = L.load()
    assert [lib.ssm_q8_num_blocks(n, 128) for n in (1, 128, 129, 1 << 40)] == [1, 1, 2, (1 << 40) // 128]
    assert lib.ssm_q8_num_blocks(0, 128) == 0 and lib.ssm_q8_num_blocks(100, 100) == 0
    assert lib.ssm_q8_num_blocks(100, 16) == 0 and lib.ssm_q8_num_blocks(100, 512) == 0


def quant(n=1000, block=128, dtype=L.SSM_BF16, x=None, q=None, s=None):
    lib = L.load()
    x = fake(0) if x is None else x
    q = fake(1) if q is None else q
    s = fake(2) if s is None else s
    return lib.ssm_q8_quantize(n, block, dtype, x, q, s, None)


def dequant(n=1000, block=128, dtype=L.SSM_BF16, parts=2, qs=None, ss=None, y=None):
    lib = L.load()
    qs = [fake(10 + i) for i in range(max(parts, 1))] if qs is None else qs
    ss = [fake(30 + i) for i in range(max(parts, 1))] if ss is None else ss
    qa = (ctypes.c_void_p * len(qs))(*[p.value if p is not None else None for p in qs])
    sa = (ctypes.c_void_p * len(ss))(*[p.value if p is not None else None for p in ss])
    y = fake(3) if y is None else y
    return lib.ssm_q8_dequant_sum(n, block, dtype, parts, qa, sa, y, None)


def test_quantize_validation():
    lib = L.load()
    assert lib.ssm_q8_quantize(10, 128, L.SSM_BF16, None, fake(1), fake(2), None) == NULL
    assert lib.ssm_q8_quantize(10, 128, L.SSM_BF16, fake(0), None, fake(2), None) == NULL
    assert lib.ssm_q8_quantize(10, 128, L.SSM_BF16, fake(0), fake(1), None, None) == NULL
    assert quant(n=0) == SHAPE and quant(n=-5) == SHAPE and quant(n=1 << 60) == SHAPE
    for b in (0, 16, 96, 100, 512):
        assert quant(block=b) == SHAPE, b
    assert quant(dtype=2) == DTYPE and quant(dtype=-1) == DTYPE
    assert quant(x=fake(0, 8)) == ALIGN      # x needs 16 bytes
    assert quant(q=fake(1, 4)) == ALIGN      # q needs 8
    assert quant(s=fake(2, 2)) == ALIGN      # scales need 4
    assert quant(q=fake(0, 1024)) == ALIAS   # q inside x (2000 bytes)
    assert quant(s=fake(0, 16)) == ALIAS     # scales inside x
    assert quant(s=fake(1, 992)) == ALIAS    # scales overlap the tail of q (1000 bytes)


def test_dequant_validation():
    lib = L.load()
    assert lib.ssm_q8_dequant_sum(10, 128, L.SSM_BF16, 1, None, None, fake(3), None) == NULL
    assert dequant(y=ctypes.c_void_p(None)) == NULL
    assert dequant(qs=[fake(10), None]) == NULL
    assert dequant(ss=[fake(30), None]) == NULL
    assert dequant(parts=0) == SHAPE and dequant(parts=17, qs=[fake(10 + i) for i in range(17)],
                                                  ss=[fake(40 + i) for i in range(17)]) == SHAPE
    assert dequant(n=0) == SHAPE and dequant(block=48) == SHAPE and dequant(dtype=7) == DTYPE
    assert dequant(y=fake(3, 8)) == ALIGN
    assert dequant(qs=[fake(10), fake(11, 4)]) == ALIGN
    assert dequant(ss=[fake(30, 2), fake(31)]) == ALIGN
    assert dequant(y=fake(11, 512)) == ALIAS      # y over part 1's codes
    assert dequant(y=fake(30, 0)) == ALIAS        # y over part 0's scales
