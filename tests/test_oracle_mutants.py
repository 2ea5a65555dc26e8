"""Plant plausible mistakes in copies of the oracle source (on the CPU) and check that
the pins catch every one of them.  The real oracle is never modified."""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssm_oracle.c")

MUTANTS = {
    "dropped_D_skip": ("r += j->Dskip[c] * u;", "r += 0.0 * u;"),
    "conv_reversed": ("w[0] * hist[0] + w[1] * hist[1] + w[2] * hist[2] + w[3] * xt",
                      "w[3] * hist[0] + w[2] * hist[1] + w[1] * hist[2] + w[0] * xt"),
    "conv_bias_dropped": ("const double bias = j->conv_b ? j->conv_b[c] : 0.0;", "const double bias = 0.0;"),
    "silu_is_sigmoid": ("const double u = v * sigmoid(v);", "const double u = sigmoid(v);"),
    "softplus_sign": ("log1p(exp(-fabs(s)))", "log1p(exp(fabs(s)))"),
    "dt_bias_dropped": ("softplus(dtr[t] + j->dt_bias[c])", "softplus(dtr[t])"),
    "A_transposed": ("exp(delta * j->A[c * N + n])", "exp(delta * j->A[n * D + c])"),
    "decay_sign": ("exp(delta * j->A[c * N + n])", "exp(-delta * j->A[c * N + n])"),
    "drive_without_delta": ("h[n] = a * h[n] + delta * Bt[n] * u;", "h[n] = a * h[n] + Bt[n] * u;"),
    "B_read_as_BNL": ("h[n] = a * h[n] + delta * Bt[n] * u;",
                      "h[n] = a * h[n] + delta * j->Bm[(b * N + n) * L + t] * u;"),
    "B_C_swapped": ("r += Ct[n] * h[n];", "r += Bt[n] * h[n];"),
    "readout_before_update": ("      h[n] = a * h[n] + delta * Bt[n] * u;\n      r += Ct[n] * h[n];",
                              "      r += Ct[n] * h[n];\n      h[n] = a * h[n] + delta * Bt[n] * u;"),
    "token_off_by_one": ("const double* Bt = j->Bm + (b * L + t) * N;",
                         "const double* Bt = j->Bm + (b * L + (t > 0 ? t - 1 : 0)) * N;"),
    "gate_without_z": ("r * zr[t] * sigmoid(zr[t])", "r * sigmoid(zr[t])"),
    "history_reversed": ("    hist[0] = hist[1];\n    hist[1] = hist[2];\n    hist[2] = xt;",
                         "    hist[2] = hist[1];\n    hist[1] = hist[0];\n    hist[0] = xt;"),
    "h0_ignored": ("h[n] = j->h0 ? j->h0[row * N + n] : 0.0;", "h[n] = 0.0;"),
    "conv0_ignored": ("if (j->conv0) memcpy(hist, j->conv0 + row * 3, sizeof hist);", ";"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) >= 1, f"mutation site for {name} no longer in the oracle source"
    mutated = source.replace(old, new, 1)
    src = tmp_path / "mutant.c"
    src.write_text(mutated)
    hdr = os.path.join(os.path.dirname(SRC), "ssm_oracle.h")
    (tmp_path / "ssm_oracle.h").write_text(open(hdr).read())
    so = tmp_path / "mutant.so"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-ffp-contract=off", "-o", str(so),
                    str(src), "-lm", "-lpthread"], check=True)
    lib = oracle.load_library(str(so))
    scan = lambda *a, **k: oracle.scan(*a, **k, lib=lib)
    failed = []
    for check_name, check in P.ALL_CHECKS.items():
        try:
            check(scan)
        except (AssertionError, FloatingPointError, ValueError, RuntimeError):
            failed.append(check_name)
    assert failed, f"mutant {name} passed every pin"
