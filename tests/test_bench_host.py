"""Host-side logic of bench.py (no GPU): the algorithmic byte and flop counts behind the reported
fractions, the parsing of rocprofv3 counter files into the traffic and issue records, and the
one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_match_the_hand_counts():
    # slice7b prefill: x, dt, z read and y written in bf16 (4 x 2 B per element over 1 x 32768 x 2048),
    # B and C once (32768 x 16 x 2 B each), final h and conv (2048 x 19 x 4 B), parameters (2048 x 23 x 4 B).
    elems = 1 * 32768 * 2048
    want = elems * 8 + 2 * 32768 * 16 * 2 + 2048 * 19 * 4 + 2048 * 23 * 4
    assert bench.prefill_bytes(1, 32768, 2048, 16, 2) == want == 539_312_128
    # decode step: per channel h and conv read + written (2 x 19 x 4 B) and x, dt, z, y (4 x 2 B);
    # parameters once; B_t and C_t once per batch row.
    assert bench.decode_bytes(1, 2048, 16, 2) == 2048 * (152 + 8) + 2048 * 23 * 4 + 2 * 16 * 2 == 516_160
    assert bench.decode_bytes(64, 5120, 16, 2) == 64 * 5120 * 160 + 5120 * 92 + 64 * 64 == 52_903_936
    # per element: conv 8, SiLU 4, softplus 4, delta*u 1, 7 per state, D-skip 2, gate 5
    assert bench.flops_per_element(16) == 136
    assert bench.flops_per_element(1) == 31


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


@pytest.fixture
def sandbox(tmp_path, monkeypatch):
    """bench.py writing its records under a scratch root, with a fixed source hash."""
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda group="scan": "h-" + group)
    return tmp_path


def test_record_traffic_scales_by_the_copy(sandbox):
    pmc = sandbox / "pmc"
    pmc.mkdir()
    gib_kib = float(1 << 20)
    copy, fill = "__amd_rocclr_copyBuffer", "fill_kernel"
    pre, dec = "prefill_windowed<bf16_t, true, 8, 8>", "decode_quad<bf16_t>"
    # The copy reads 1 GiB and writes 1 GiB; its FETCH_SIZE counter reads half (a 2x scale), its
    # WRITE_SIZE in full.  A fill writes 1 GiB and reads nothing; it must not be taken as the copy.
    fetch = [(1, fill, 0.0), (2, copy, gib_kib / 2), (3, pre, 1000.0), (4, pre, 1002.0), (5, dec, 10.0)]
    write = [(1, fill, gib_kib), (2, copy, gib_kib), (3, pre, 500.0), (4, pre, 500.0), (5, dec, 8.0)]
    for ctr, vals in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
        _write_csv(pmc / f"{ctr}_counter_collection.csv",
                   [{"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": ctr, "Counter_Value": v} for d, k, v in vals])
    bench.record_traffic(str(pmc), "slice7b")
    rec = json.load(open(sandbox / "profiles" / "traffic.json"))["slice7b"]
    assert rec["copy_calibration"]["kernel"] == copy
    assert rec["copy_calibration"]["fetch_scale"] == 2.0 and rec["copy_calibration"]["write_scale"] == 1.0
    assert rec["prefill"]["dispatches"] == 2
    assert rec["bytes_per_launch"] == int((1001.0 * 2 + 500.0) * 1024)
    assert rec["decode"]["bytes_per_launch"] == int((10.0 * 2 + 8.0) * 1024)
    assert rec["source_hash"] == "h-scan"
    assert bench.traffic_from_profiles("slice7b") == rec["bytes_per_launch"]
    assert bench.traffic_from_profiles("slice7b", "decode") == rec["decode"]["bytes_per_launch"]


def test_traffic_record_void_when_sources_change(sandbox, monkeypatch):
    rec = {"slice7b": {"sources": "scan", "source_hash": "h-scan", "bytes_per_launch": 123}}
    (sandbox / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert bench.traffic_from_profiles("slice7b") == 123
    monkeypatch.setattr(bench, "kernel_source_hash", lambda group="scan": "changed")
    assert bench.traffic_from_profiles("slice7b") is None
    assert bench.traffic_from_profiles("mamba2.8b") is None


def test_record_issue_leaves_out_the_warmup_dispatch(sandbox):
    path = sandbox / "sq_counter_collection.csv"
    k = "prefill_windowed<bf16_t, true, 8, 8>"
    waves = 2048
    rows = []
    # dispatch 7 is the warm-up (slower); 8 and 9 are the timed calls; a decode dispatch is ignored
    for d, cycles in ((7, 250_000.0), (8, 224_000.0), (9, 226_000.0)):
        for ctr, per_wave in (("SQ_WAVES", 1.0), ("SQ_WAVE_CYCLES", cycles), ("SQ_ACTIVE_INST_VALU", 99_000.0),
                              ("SQ_INSTS_VALU", 87_000.0)):
            # counters arrive split over several rows (per XCD); the parser sums them
            for part in (0.25, 0.75):
                rows.append({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": ctr,
                             "Counter_Value": per_wave * waves * part})
    rows.append({"Dispatch_Id": 10, "Kernel_Name": "decode_quad<bf16_t>", "Counter_Name": "SQ_WAVES",
                 "Counter_Value": 32.0})
    _write_csv(path, rows)
    bench.record_issue(str(path), "slice7b")
    issue = json.load(open(sandbox / "profiles" / "traffic.json"))["slice7b"]["issue"]
    assert issue["dispatches"] == 2 and issue["warmup_dispatches_left_out"] == 1
    assert issue["waves"] == waves
    assert issue["wave_cycles_per_wave"] == 225_000.0
    # each of the 1024 SIMDs holds two waves: busy = 2 x active / cycles
    assert issue["valu_issue_busy"] == round(2 * 99_000.0 / 225_000.0, 4)
    assert bench.issue_from_profiles("slice7b") == issue


def test_valu_roofline_arithmetic():
    """plain = insts - trans, trans = active - insts; t_min = waves x (plain / R_plain + trans /
    R_trans) slots at 1024 SIMDs x 2.4 GHz / 4; frac = t_min / kernel time."""
    issue = {"waves": 2048, "insts_valu_per_wave": 90_000.0, "active_inst_valu_per_wave": 100_000.0,
             "valu_issue_busy": 0.9}
    cal = {"issue": [{"kind": k, "waves_per_simd": w, "inst_per_slot_median": r}
                     for k, pts in (("fma", ((1, 0.75), (2, 1.5), (4, 1.6))), ("exp", ((1, 0.44), (2, 0.5), (4, 0.5))))
                     for w, r in pts]}
    r = bench.valu_roofline(issue, cal, 0.5)
    assert r["waves_per_simd"] == 2.0 and r["trans_per_wave"] == 10_000.0
    assert r["rates_inst_per_slot"] == {"plain": 1.5, "trans": 0.5, "at_waves_per_simd": 2}
    t_min = 2048 * (80_000 / 1.5 + 10_000 / 0.5) / (1024 * 2.4e9 / 4)
    assert r["t_min_ms"] == round(t_min * 1e3, 4)
    assert r["frac"] == round(t_min / 0.5e-3, 4)
    assert r["achieved"] == round(2048 * 90_000 * 64 / 0.5e-3 / 1e12, 3)
    assert r["peak"] == round(2048 * 90_000 * 64 / t_min / 1e12, 3)
    assert bench.valu_roofline(None, cal, 0.5)["achieved"] is None
    assert bench.valu_roofline(issue, None, 0.5)["frac"] is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
