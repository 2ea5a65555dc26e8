"""Rate calibration of the GPU the scan runs on (include/ssm_calib.h).

    python -m selective_state_space_causal_amd.calib [--json profiles/calib.json] [--md profiles/calib_mi355x.md]

Measures, on the device itself:
  * vector-instruction issue: fp32 FMA, the v_exp_f32 transcendental, and a 4 : 1 mix of the two,
    each at 1, 2, 3, 4 and 8 waves per SIMD; other single-instruction mixes (v_mul_f32, v_fmac_f32,
    three-source v_fma_f32, DPP v_fmac_f32), the 4 : 1 mix with independent exp chains, and SIMDs
    holding one FMA wave beside one exp wave, at fewer occupancies.  Every wave stamps its start and end on the shader
    clock (s_memtime) and on the constant 100 MHz clock (s_memrealtime) and records which SIMD ran
    it (HW_ID, XCC_ID), so the rate comes out per SIMD and per clock cycle, with the placement of
    the waves checked rather than assumed, and the clock the SIMDs ran at comes out too;
  * plain HBM streams: a 1 GiB device copy (read + write) and a 1 GiB read.

The issue rate is reported as instructions per SIMD per 4-cycle issue slot (a wave64 VALU
instruction occupies its SIMD's 16-lane ALU for 4 cycles): 1.0 is one instruction per slot.
The prefill scan's roofline (bench.py) divides the VALU issue slots its counters record by the
slots this calibration shows the SIMDs can fill at the scan's waves per SIMD.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
from collections import defaultdict

import torch

from . import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KINDS = dict(L.CALIB_KINDS)
# Per wave and loop iteration (ssm_calib.hip: 8 chains, unrolled by 4): (plain, transcendental)
# instructions of each mix; under "split" a wave runs fma or exp.
PER_ITER = {"fma": (32, 0), "exp": (0, 32), "mix": (128, 32), "mul": (32, 0), "fmac": (32, 0), "fma3": (32, 0),
            "dpp": (32, 0), "mixi": (128, 32)}
KIND_NAMES = {v: k for k, v in KINDS.items()}
WAVES = (1, 2, 3, 4, 8)
REALTIME_HZ = 100e6  # s_memrealtime


def source_hash() -> str:
    """Identifies the measurement: the microbenchmark kernels and the code that turns their
    stamps into rates (a record stays valid while both are unchanged)."""
    import inspect

    h = hashlib.sha256(open(os.path.join(ROOT, "selective_state_space_causal_amd/csrc/ssm_calib.hip"), "rb").read())
    for fn in (issue_point, stream_rates, decode_hw_id):
        h.update(inspect.getsource(fn).encode())
    h.update(repr(sorted(PER_ITER.items())).encode())
    return h.hexdigest()[:16]


def decode_hw_id(hw: int, xcc: int):
    """(xcc, se, sh, cu, simd) of a wave from its HW_ID / XCC_ID registers (gfx9 layout:
    SIMD_ID bits 5:4, CU_ID 11:8, SH_ID 12, SE_ID 15:13)."""
    return (xcc & 0xF, (hw >> 13) & 7, (hw >> 12) & 1, (hw >> 8) & 0xF, (hw >> 4) & 3)


def issue_point(kind: str, waves_per_simd: int, iters: int, cus: int):
    """One launch of `kind` at `waves_per_simd`; rates per SIMD from the waves' shader-clock
    stamps.  inst_per_slot counts instructions; slot_units_per_slot counts a transcendental as
    two (the unit SQ_ACTIVE_INST_VALU counts in)."""
    wg = cus * waves_per_simd
    split = wg // 2 if kind == "split" else 0  # first half of the workgroups: fma, second half: exp
    L.calib_issue(KINDS[kind], wg, max(1, iters // 8), split)  # warm-up (code, clocks)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    stamps, _ = L.calib_issue(KINDS[kind], wg, iters, split)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    st = stamps.cpu().tolist()
    per_simd = defaultdict(list)
    freqs = []
    for t0, t1, r0, r1, hw, xcc, ran, _ in st:
        plain, trans = PER_ITER[KIND_NAMES[ran]]
        per_simd[decode_hw_id(hw, xcc)].append((t0, t1, iters * plain, iters * trans, KIND_NAMES[ran]))
        if r1 > r0:
            freqs.append((t1 - t0) / ((r1 - r0) / REALTIME_HZ))
    rates, units, counts, mixed = [], [], [], defaultdict(list)
    total_insts = 0
    for waves in per_simd.values():
        counts.append(len(waves))
        span = (max(w[1] for w in waves) - min(w[0] for w in waves)) / 4.0  # issue slots the SIMD was busy
        insts = sum(w[2] + w[3] for w in waves)
        total_insts += insts
        rates.append(insts / span)
        units.append(sum(w[2] + 2 * w[3] for w in waves) / span)
        if len({w[4] for w in waves}) > 1:  # split: this SIMD held waves of both mixes
            for w in waves:
                mixed[w[4]].append((w[2] + w[3]) / ((w[1] - w[0]) / 4.0))
    med = statistics.median
    out = {"kind": kind, "waves_per_simd": waves_per_simd, "workgroups": wg, "iters": iters,
           "simds_used": len(per_simd), "waves_per_simd_seen": [min(counts), max(counts)],
           "inst_per_slot_median": round(med(rates), 4),
           "inst_per_slot_min": round(min(rates), 4), "inst_per_slot_max": round(max(rates), 4),
           "slot_units_per_slot_median": round(med(units), 4),
           "lane_ops_per_clk_per_cu": round(med(rates) * 64, 2),
           "shader_ghz_median": round(med(freqs) / 1e9, 3), "kernel_ms": round(ms, 4),
           "lane_ops_per_s_T": round(total_insts * 64 / (ms * 1e-3) / 1e12, 3)}
    if mixed:
        out["split_simds"] = len(mixed.get("fma", []))
        out["split_wave_inst_per_slot"] = {k: round(med(v), 4) for k, v in mixed.items()}
    return out


def stream_rates(nbytes: int = 1 << 30, reps: int = 5):
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    sink = L.calib_read(src)
    out = {}
    for name, fn, moved in (("copy", lambda: L.calib_copy(src, dst), 2 * nbytes),
                            ("read", lambda: L.calib_read(src, sink), nbytes)):
        fn()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = statistics.median(times)
        out[name] = {"bytes_moved": moved, "ms_median": round(ms, 4), "gbps": round(moved / (ms * 1e-3) / 1e9, 1)}
    return out


def run(iters: int = 4096):
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    points = [issue_point(k, w, iters, cus) for k in ("fma", "exp", "mix") for w in WAVES]
    points += [issue_point(k, w, iters, cus) for k in ("mul", "fmac", "fma3", "dpp", "mixi") for w in (1, 2, 4)]
    points += [issue_point("split", w, iters, cus) for w in (2, 4)]
    return {"device": props.name, "gcn_arch": getattr(props, "gcnArchName", ""), "cus": cus,
            "source_hash": source_hash(), "issue": points, "streams": stream_rates()}


def markdown(rec, command):
    out = [f"# Rate calibration: {rec['device']} ({rec['gcn_arch']}, {rec['cus']} CUs)", "",
           "Produced by:", "", "```", command, "```", "",
           "Issue rate = instructions per SIMD per 4-cycle issue slot, from each wave's shader-clock stamps and the "
           "SIMD it ran on (median over SIMDs; min-max beside it). A transcendental that holds two slots shows as "
           "0.5 when issued alone.", "",
           "| mix | waves/SIMD (seen) | inst/slot median | min-max | slot units/slot | lane-ops/clk/CU | shader GHz | "
           "T lane-ops/s |",
           "|---|---|---|---|---|---|---|---|"]
    for p in rec["issue"]:
        seen = p["waves_per_simd_seen"]
        out.append(f"| {p['kind']} | {p['waves_per_simd']} ({seen[0]}-{seen[1]}) | {p['inst_per_slot_median']:.3f} | "
                   f"{p['inst_per_slot_min']:.3f}-{p['inst_per_slot_max']:.3f} | {p['slot_units_per_slot_median']:.3f} | "
                   f"{p['lane_ops_per_clk_per_cu']:.1f} | {p['shader_ghz_median']:.3f} | {p['lane_ops_per_s_T']:.2f} |")
    splits = [p for p in rec["issue"] if "split_wave_inst_per_slot" in p]
    if splits:
        out += ["", "Split: SIMDs that held one fma wave and one exp wave at once, each wave's own rate "
                "(instructions per slot of its lifetime):", "",
                "| waves/SIMD | SIMDs with both | fma wave | exp wave |", "|---|---|---|---|"]
        for p in splits:
            r = p["split_wave_inst_per_slot"]
            out.append(f"| {p['waves_per_simd']} | {p['split_simds']} | {r.get('fma', 0):.3f} | {r.get('exp', 0):.3f} |")
    s = rec["streams"]
    out += ["", "| stream | bytes moved | ms (median of 5) | GB/s |", "|---|---|---|---|"]
    for k, v in s.items():
        out.append(f"| {k} | {v['bytes_moved']} | {v['ms_median']} | {v['gbps']} |")
    return "\n".join(out) + "\n"


def rate(rec, kind: str, waves_per_simd: int) -> float:
    """The measured issue rate of one mix (instructions per SIMD per slot) at the calibrated
    occupancy nearest `waves_per_simd`, from a calibration record."""
    pts = [p for p in rec["issue"] if p["kind"] == kind]
    best = min(pts, key=lambda p: abs(p["waves_per_simd"] - waves_per_simd))
    return best["inst_per_slot_median"]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--json", default=None, help="write the record here (e.g. profiles/calib.json)")
    ap.add_argument("--md", default=None, help="write the markdown summary here")
    ap.add_argument("--iters", type=int, default=4096)
    args = ap.parse_args()
    rec = run(args.iters)
    cmd = "python -m selective_state_space_causal_amd.calib" + \
        (f" --json {args.json}" if args.json else "") + (f" --md {args.md}" if args.md else "") + \
        (f" --iters {args.iters}" if args.iters != 4096 else "")
    rec["command"] = cmd
    md = markdown(rec, cmd)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    if args.md:
        with open(args.md, "w") as f:
            f.write(md)
    print(md)


if __name__ == "__main__":
    main()
