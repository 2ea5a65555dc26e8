"""Plant plausible mistakes in copies of the projection oracle (on the CPU) and check that
the pins catch every one of them.  The real oracle is never modified."""
import importlib.util

import pytest

from oracle import proj
from tests import proj_pins as P

MUTANTS = {
    "in_proj_token_major_out": ('np.einsum("blk,ck->bcl"', 'np.einsum("blk,ck->blc"'),
    "in_proj_weight_transposed": ('np.einsum("blk,ck->bcl"', 'np.einsum("blk,kc->bcl"'),
    "x_proj_channel_major_out": ('np.einsum("bcl,jc->blj"', 'np.einsum("bcl,jc->bjl"'),
    "x_proj_weight_transposed": ('np.einsum("bcl,jc->blj"', 'np.einsum("bcl,cj->blj"'),
    "dt_proj_weight_transposed": ('np.einsum("blr,cr->bcl"', 'np.einsum("blr,rc->bcl"'),
    "out_proj_weight_transposed": ('np.einsum("bcl,mc->blm"', 'np.einsum("bcl,cm->blm"'),
    "conv_reversed": ("xi[:, :, k:k + L]", "xi[:, :, 3 - k:3 - k + L]"),
    "conv_bias_dropped": ("v = np.zeros((B, D, L)) if conv_b is None else", "v = np.zeros((B, D, L)) if True else"),
    "conv0_ignored": ("hist = np.zeros((B, D, 3)) if conv0 is None else _f64(conv0)", "hist = np.zeros((B, D, 3))"),
    "silu_is_sigmoid": ("return v / (1.0 + np.exp(-v))", "return 1.0 / (1.0 + np.exp(-v))"),
    "history_reversed": ("xi = np.concatenate([hist, x], axis=2)", "xi = np.concatenate([hist[:, :, ::-1], x], axis=2)"),
    "decode_conv_cache_ignored": ('u = to_io(conv_silu(x, params["conv_w"], params.get("conv_b"), _f64(conv)), io)',
                                  'u = to_io(conv_silu(x, params["conv_w"], params.get("conv_b")), io)'),
    "decode_gate_from_x": ('z = to_io(in_proj(hid, w["in_z"]), io)', 'z = to_io(in_proj(hid, w["in_x"]), io)'),
    "decode_B_C_swapped": ('tok = {"x": x[..., 0], "dt": dt[..., 0], "z": z[..., 0], "Bm": Bm[:, 0], "Cm": Cm[:, 0]}',
                           'tok = {"x": x[..., 0], "dt": dt[..., 0], "z": z[..., 0], "Bm": Cm[:, 0], "Cm": Bm[:, 0]}'),
    "decode_dt_unrounded": ('dt = to_io(dt_proj(lowrank, w["dt"]), io)                          # [B, D, 1]',
                            'dt = dt_proj(lowrank, w["dt"])                                     # [B, D, 1]'),
}


@pytest.fixture(scope="module")
def source():
    with open(proj.__file__) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_proj_pins_catch_mutant(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) >= 1, f"mutation site for {name} no longer in the projection oracle"
    path = tmp_path / "proj_mutant.py"
    path.write_text(source.replace(old, new, 1))
    # named inside the oracle package, so that its layer compositions reach the scan oracle
    spec = importlib.util.spec_from_file_location("oracle.proj_mutant", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for check_name, check in P.ALL_CHECKS.items():
        try:
            check(mod)
        except (AssertionError, ValueError, IndexError, RuntimeError):
            failed.append(check_name)
    assert failed, f"mutant {name} passed every pin"
