"""C ABI of the rate calibration (include/ssm_calib.h) without a GPU: exports and host-side
validation.  Every call below is invalid on purpose and must be rejected before any HIP call,
so the fake device addresses are never used."""
import ctypes
import os
import re

import pytest
import torch

from selective_state_space_causal_amd import _lib as L

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake-pointer tests run only without a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_calib.h")
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced
NULL, SHAPE, ALIGN, ALIAS = 1, 2, 4, 5


def test_exports_every_declared_symbol():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(ssm_[a-z_]+)\s*\(", src)))
    assert {"ssm_calib_issue", "ssm_calib_copy", "ssm_calib_read", "ssm_calib_read_sink_floats"} <= set(names)
    lib = L.load()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ssm_calib.h but not exported"


def test_issue_validation():
    lib = L.load()
    assert lib.ssm_calib_issue(0, 4, 8, 0, None, FAKE, None) == NULL
    assert lib.ssm_calib_issue(0, 4, 8, 0, FAKE, None, None) == NULL
    assert lib.ssm_calib_issue(9, 4, 8, 0, FAKE, FAKE, None) == SHAPE      # unknown mix
    assert lib.ssm_calib_issue(-1, 4, 8, 0, FAKE, FAKE, None) == SHAPE
    assert lib.ssm_calib_issue(0, 0, 8, 0, FAKE, FAKE, None) == SHAPE      # no workgroup
    assert lib.ssm_calib_issue(0, 4, 0, 0, FAKE, FAKE, None) == SHAPE      # no iteration
    assert lib.ssm_calib_issue(0, (1 << 20) + 1, 8, 0, FAKE, FAKE, None) == SHAPE


def test_stream_validation():
    lib = L.load()
    assert lib.ssm_calib_copy(None, FAKE, 16, None) == NULL
    assert lib.ssm_calib_copy(FAKE, FAKE + 4096, 0, None) == SHAPE
    assert lib.ssm_calib_copy(FAKE, FAKE + 4096, 24, None) == SHAPE
    assert lib.ssm_calib_copy(FAKE + 4, FAKE + 4096, 16, None) == ALIGN
    assert lib.ssm_calib_copy(FAKE, FAKE + 16, 64, None) == ALIAS
    assert lib.ssm_calib_read(None, 16, FAKE, None) == NULL
    assert lib.ssm_calib_read(FAKE, 16, None, None) == NULL
    assert lib.ssm_calib_read(FAKE, 8, FAKE + 4096, None) == SHAPE
    assert lib.ssm_calib_read(FAKE + 8, 16, FAKE + 4096, None) == ALIGN
    assert lib.ssm_calib_read_sink_floats() >= 1


def test_hw_id_decoding():
    from selective_state_space_causal_amd.calib import decode_hw_id
    # SIMD 2, CU 9, SH 1, SE 5 on XCD 6
    hw = (2 << 4) | (9 << 8) | (1 << 12) | (5 << 13) | 0x3
    assert decode_hw_id(hw, 6) == (6, 5, 1, 9, 2)
