"""Plant plausible mistakes in copies of the codec oracle (on the CPU) and check that the
pins catch every one of them.  The real oracle is never modified."""
import importlib.util
import os

import pytest

from oracle import codec
from tests import codec_pins as P

SRC = codec.__file__

MUTANTS = {
    "divides_by_128": ("safe / np.float32(QMAX)", "safe / np.float32(128)"),
    "multiplier_128": ("np.float32(QMAX) / safe", "np.float32(128) / safe"),
    "amax_signed": ("amax = np.abs(xb).max(axis=1)", "amax = xb.max(axis=1)"),
    "round_half_up": ("codes = np.rint(xb * inv[:, None])", "codes = np.floor(xb * inv[:, None] + 0.5)"),
    "truncate": ("codes = np.rint(xb * inv[:, None])", "codes = np.trunc(xb * inv[:, None])"),
    "zero_block_scale_one": ("np.where(nonzero, safe / np.float32(QMAX), np.float32(0))",
                             "np.where(nonzero, safe / np.float32(QMAX), np.float32(1))"),
    "one_scale_per_tensor": ("amax = np.abs(xb).max(axis=1)",
                             "amax = np.full(xb.shape[0], np.abs(xb).max(), np.float32)"),
    "owner_modulo": ("owner = np.arange(n) // block", "owner = np.arange(n) % block % scales.shape[1]"),
    "first_part_only": ("for p in range(parts):", "for p in range(1):"),
    "part0_scales": ("scales[p, owner]", "scales[0, owner]"),
    "clamp_126": ("codes = np.clip(codes, -QMAX, QMAX)", "codes = np.clip(codes, -QMAX + 1, QMAX - 1)"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_codec_pins_catch_mutant(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) >= 1, f"mutation site for {name} no longer in the codec oracle"
    path = tmp_path / "codec_mutant.py"
    path.write_text(source.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("codec_mutant", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for check_name, check in P.ALL_CHECKS.items():
        try:
            check(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(check_name)
    assert failed, f"mutant {name} passed every pin"
