"""The rate calibration's kernels on the GPU: stamps and placement are recorded for every wave,
the copy stream copies, and the read stream covers every byte (needs an MI355X)."""
import pytest
import torch

from selective_state_space_causal_amd import _lib as L
from selective_state_space_causal_amd import calib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["fma", "exp", "mix"])
def test_issue_point_records_every_wave(kind):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    p = calib.issue_point(kind, 2, 64, cus)
    assert p["simds_used"] >= 4 * cus * 0.9            # waves spread over (nearly) every SIMD
    assert p["waves_per_simd_seen"][1] <= 4
    assert 0.05 < p["inst_per_slot_median"] <= 2.0
    assert 0.5 < p["shader_ghz_median"] < 4.0


def test_copy_and_read_streams():
    n = (1 << 20) + 4
    src = torch.randn(n, device="cuda")
    dst = torch.zeros_like(src)
    L.calib_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    ones = torch.full((4096 * 4,), 1.0, device="cuda")      # 16 KiB of 0x3f800000 words
    sink = L.calib_read(ones)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
