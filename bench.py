#!/usr/bin/env python3
"""Benchmark of the selective-SSM hot path on one MI355X.

One step = one ssm_prefill over the workload's prompt (which leaves the h / conv cache)
followed by its decode steps (one ssm_decode_step per token, each resuming from the cache).
Inputs are synthetic and already resident in HBM when the timed region starts.

Prints ONE JSON line: value = prefill Gelem/s over B*L*d_inner; decode_us_per_step is the
mean decode-step time; roofline describes the prefill kernel; cpu_baseline is the fp64
oracle timed on this host's cores on the same input bits.  decode_at_scale times the decode
step on the mamba2.8b cache (batch 64, d_inner 5120), where it is bound by HBM rather than by
launch latency.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD public specification
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, AMD public specification
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, AMD public specification
CONV_W = 4


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class TimingEvent:
    """A HIP event for timing only, recorded on an explicit stream.  It is created with
    hipEventDisableSystemFence: recording it does not flush the caches for host visibility,
    which a default event does and which would add ~20 us to a single prefill that no
    pipeline pays.  Falls back to a torch.cuda.Event when the flag is not available."""

    _hip = None
    FLAG = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        import torch

        self.ct = ctypes
        if TimingEvent._hip is None:
            try:
                TimingEvent._hip = ctypes.CDLL("libamdhip64.so")
            except OSError:
                TimingEvent._hip = False
        self.handle = None
        if TimingEvent._hip:
            h = ctypes.c_void_p()
            if TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(h), self.FLAG) == 0:
                self.handle = h
        self.fallback = None if self.handle is not None else torch.cuda.Event(enable_timing=True)

    def record(self, stream):
        if self.fallback is not None:
            self.fallback.record(stream)
        else:
            TimingEvent._hip.hipEventRecord(self.handle, self.ct.c_void_p(stream.cuda_stream))

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both completed)."""
        if self.fallback is not None:
            return self.fallback.elapsed_time(end.fallback)
        ms = self.ct.c_float()
        TimingEvent._hip.hipEventElapsedTime(self.ct.byref(ms), self.handle, end.handle)
        return ms.value

    def __del__(self):
        if self.handle is not None and TimingEvent._hip:
            TimingEvent._hip.hipEventDestroy(self.handle)


def flops_per_element(N: int) -> int:
    """Algorithmic fp32 operations per (b, c, t) element, a transcendental counted as one:
    conv 4 FMA (8); SiLU exp+add+rcp+mul (4); softplus add+exp+add+log (4); delta*u (1);
    per state: delta*A, exp, (delta u)*B, FMA h, FMA y (7); D-skip FMA (2); gate (5)."""
    return 8 + 4 + 4 + 1 + 7 * N + 2 + 5


def prefill_bytes(B, L, D, N, es):
    """Algorithmic HBM bytes of one prefill: read x, dt, z and write y once; B and C once;
    final h and conv (fp32); per-channel parameters."""
    return B * D * L * 4 * es + B * L * 2 * N * es + B * D * (N + CONV_W - 1) * 4 + D * (N + 7) * 4


def decode_bytes(B, D, N, es):
    """Algorithmic HBM bytes of one decode step: h and conv read + written (fp32), x, dt, z
    read and y written, parameters, B_t and C_t."""
    return B * D * (2 * (N + CONV_W - 1) * 4 + 4 * es) + D * (N + 7) * 4 + B * 2 * N * es


def timed_steps(step, nevents, warmup, steps):
    """Run `warmup` untimed calls of step(events), then `steps` timed ones between
    torch.cuda.synchronize() calls.  Every call's HIP events are created before the first call
    and Python's garbage collector is paused meanwhile, so no host-side stall (an event
    creation, a collection) can fall between two recorded events while the GPU waits for the
    next launch.  Returns (the timed calls' events, wall seconds of the timed calls)."""
    import gc

    import torch

    evs = [[TimingEvent() for _ in range(nevents)] for _ in range(warmup + steps)]
    gc.collect()
    gc.disable()
    try:
        for i in range(warmup):
            step(evs[i])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(warmup, warmup + steps):
            step(evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    finally:
        gc.enable()
    return evs[warmup:], t1 - t0


# The sources each measured kernel is built from: a traffic record stays valid while these
# files are unchanged (a change elsewhere in the library does not touch that kernel).
KERNEL_SOURCES = {
    "scan": ["ssm_windowed.hip", "ssm_decode.hip", "ssm_decode_quad.h", "ssm_seq.hip", "ssm_device.h", "ssm_internal.h"],
    "codec": ["ssm_codec.hip", "ssm_device.h"],
}


def kernel_source_hash(group="scan"):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[group]:
        f = os.path.join(ROOT, "selective_state_space_causal_amd", "csrc", name)
        h.update(name.encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload, kernel=None):
    """HBM traffic per launch (of the prefill kernel, or of `kernel`'s entry) from the committed
    rocprofv3 --pmc summary, or None when there is none for this workload or the kernels
    changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(rec.get("sources", "scan")):
        return None
    if kernel is not None:
        return (rec.get(kernel) or {}).get("bytes_per_launch")
    return rec.get("bytes_per_launch")


PMC_COMMAND = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {ctr} -d $REPO/gpurun_out/pmc -o {ctr} "
               "--output-format csv -- python3 $REPO/bench.py --steps 2 --warmup 1 --no-cpu-baseline "
               "--decode-steps 8 --copy-calibration --workload {workload}")
PMC_COMMAND_DECODE = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {ctr} -d $REPO/gpurun_out/pmc_{scale} -o {ctr} "
                      "--output-format csv -- python3 $REPO/bench.py --decode-at-scale-only {scale} --steps 2 "
                      "--warmup 1")
PMC_COMMAND_CODEC = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {ctr} -d $REPO/gpurun_out/pmc_codec -o {ctr} "
                     "--output-format csv -- python3 $REPO/bench.py --codec {workload} --steps 2 --warmup 1 "
                     "--no-cpu-baseline --copy-calibration")


SQ_COMMAND = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY "
              "SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU SQ_INSTS_VALU -d $REPO/gpurun_out/pmcsq -o {tag} "
              "--output-format csv -- python3 $REPO/bench.py --workload {workload} --steps 2 --warmup 1 "
              "--no-cpu-baseline --decode-steps 0")
MI355X_SIMDS = 256 * 4


def record_issue(csv_path, workload):
    """Add the prefill kernel's VALU issue occupancy to profiles/traffic.json, from one
    rocprofv3 --pmc run holding SQ_WAVES, SQ_WAVE_CYCLES and SQ_ACTIVE_INST_VALU (4-cycle units,
    summed over waves): the share of each SIMD's issue slots, over the kernel's duration, in
    which one of its waves issued a VALU instruction (a transcendental holds two slots).  The
    kernel's duration is taken as a wave's lifetime, which holds when every wave is resident
    from start to end (one round, as for slice7b's 2048 waves on 1024 SIMDs).  The run's first
    prefill dispatch is its warm-up call, which bench.py also leaves out of its timing (it runs
    ~8% longer, on caches and translations not yet warm): it is left out here too."""
    import csv
    from collections import defaultdict

    per = defaultdict(lambda: defaultdict(float))
    name = None
    for r in csv.DictReader(open(csv_path)):
        if "prefill_" not in r["Kernel_Name"]:
            continue
        name = r["Kernel_Name"]
        per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no prefill dispatch in {csv_path}")
    order = sorted(per, key=int)
    if len(order) > 1:
        per = {k: per[k] for k in order[1:]}
    mean = lambda k: sum(d[k] for d in per.values()) / len(per)
    waves, cycles, active = mean("SQ_WAVES"), mean("SQ_WAVE_CYCLES"), mean("SQ_ACTIVE_INST_VALU")
    if waves > MI355X_SIMDS * 2:
        raise SystemExit("more than two waves per SIMD: waves are not all resident at once")
    issue = {"kernel": name, "dispatches": len(per), "warmup_dispatches_left_out": len(order) - len(per),
             "source_hash": kernel_source_hash("scan"),
             "command": SQ_COMMAND.format(tag=os.path.basename(csv_path).split("_counter")[0], workload=workload),
             "waves": int(waves), "wave_cycles_per_wave": round(cycles / waves, 1),
             "active_inst_valu_per_wave": round(active / waves, 1),
             "insts_valu_per_wave": round(mean("SQ_INSTS_VALU") / waves, 1),
             "valu_issue_busy": round(active / (MI355X_SIMDS * cycles / waves), 4)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    rec.setdefault(workload, {})["issue"] = issue
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(issue, indent=1))


def issue_from_profiles(workload):
    """The prefill kernel's recorded VALU issue counters (record_issue), or None (no record, or
    the kernel sources changed since they were taken)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = (json.load(open(path)).get(workload) or {}).get("issue")
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash("scan"):
        return None
    return rec


def calib_from_profiles():
    """The committed rate calibration (profiles/calib.json, written by
    python -m selective_state_space_causal_amd.calib), or None when it is missing or its
    microbenchmarks changed since it was taken."""
    from selective_state_space_causal_amd import calib

    path = os.path.join(ROOT, "profiles", "calib.json")
    try:
        rec = json.load(open(path))
    except (ValueError, OSError):
        return None
    return rec if rec.get("source_hash") == calib.source_hash() else None


# The vector ALUs of an MI355X (AMD public specification): 256 CUs of 4 SIMDs, each SIMD 16
# lanes wide, at 2.4 GHz; a wave64 VALU instruction is issued to its SIMD in a 4-cycle slot.
# How many instructions a SIMD completes per slot depends on the instruction and on the waves
# it holds, and is measured (selective_state_space_causal_amd.calib): at two waves per SIMD,
# plain fp32 arithmetic reaches ~1.5 per slot (two waves issue in the same slot) and v_exp_f32
# ~0.47 (a transcendental holds the SIMD for two slots and is not paired).
MI355X_CUS, SIMDS_PER_CU, SIMD_LANES, CLOCK_HZ = 256, 4, 16, 2.4e9
SLOTS_PER_S = MI355X_CUS * SIMDS_PER_CU * CLOCK_HZ / 4  # per SIMD-slot, chip-wide


def valu_roofline(issue, cal, kernel_ms):
    """Issue roofline of the prefill kernel (bound "alu").  From the committed counters, per
    wave: SQ_INSTS_VALU = plain + transcendental instructions and SQ_ACTIVE_INST_VALU = plain +
    2 x transcendental slots, so trans = active - insts and plain = insts - trans.  The kernel's
    shortest possible duration at the calibrated rates (plain at the fp32 FMA rate, trans at the
    v_exp_f32 rate, both per SIMD per slot at the kernel's waves per SIMD) is
        t_min = waves x (plain / R_plain + trans / R_trans) / (1024 SIMDs x 0.6e9 slots/s),
    the rates' slots taken at the published 2.4 GHz.  achieved = all VALU lane-operations /
    the measured kernel time; peak = the same operations / t_min; frac = t_min / time.  DPP
    instructions count as plain although they do not pair (measured ~0.9 per slot), so the
    peak is on the high side.  Null where the counters or the calibration are stale or
    missing."""
    out = {"bound": "alu", "unit": "T lane-ops/s", "achieved": None, "peak": None, "frac": None,
           "valu_insts_per_wave": None, "trans_per_wave": None, "waves_per_simd": None,
           "rates_inst_per_slot": None, "valu_issue_busy": None}
    if issue is None:
        return out
    from selective_state_space_causal_amd import calib

    waves = issue["waves"]
    wps = waves / (MI355X_CUS * SIMDS_PER_CU)
    insts = issue["insts_valu_per_wave"]
    trans = issue["active_inst_valu_per_wave"] - insts
    plain = insts - trans
    lane_ops = waves * insts * 64
    out.update({"achieved": round(lane_ops / (kernel_ms * 1e-3) / 1e12, 3), "valu_insts_per_wave": insts,
                "trans_per_wave": round(trans, 1), "waves_per_simd": round(wps, 3),
                "valu_issue_busy": issue.get("valu_issue_busy")})
    if cal is not None:
        w = max(1, round(wps))
        rp, rt = calib.rate(cal, "fma", w), calib.rate(cal, "exp", w)
        t_min = waves * (plain / rp + trans / rt) / SLOTS_PER_S
        out.update({"rates_inst_per_slot": {"plain": rp, "trans": rt, "at_waves_per_simd": w},
                    "t_min_ms": round(t_min * 1e3, 4), "peak": round(lane_ops / t_min / 1e12, 3),
                    "frac": round(t_min / (kernel_ms * 1e-3), 4)})
    return out


def record_traffic(pmc_dir, workload):
    """Turn the two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) into
    profiles/traffic.json.  Each counter is scaled by what it reads for the plain 1 GiB copy
    run in the same process (--copy-calibration): 1 GiB read and 1 GiB written."""
    import csv
    from collections import defaultdict

    per = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = list(csv.DictReader(open(os.path.join(pmc_dir, f"{ctr}_counter_collection.csv"))))
        vals = defaultdict(list)
        for r in rows:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        per[ctr] = vals
    gib_kib = float(1 << 20)
    # The calibration copy is the device-to-device copy dispatch that writes a full GiB (the
    # fill that initialises its source writes a GiB too but reads nothing).
    copies = [k for k in per["WRITE_SIZE"] if "copyBuffer" in k] or list(per["WRITE_SIZE"])
    copy_name = max(copies, key=lambda k: max(per["WRITE_SIZE"][k]) + max(per["FETCH_SIZE"].get(k, [0.0])))
    wi = per["WRITE_SIZE"][copy_name].index(max(per["WRITE_SIZE"][copy_name]))
    fetch_scale = gib_kib / per["FETCH_SIZE"][copy_name][wi]
    write_scale = gib_kib / per["WRITE_SIZE"][copy_name][wi]

    def kernel(tag):
        names = [k for k in per["FETCH_SIZE"] if tag in k]
        if not names:
            return None
        k = names[0]
        f = sum(per["FETCH_SIZE"][k]) / len(per["FETCH_SIZE"][k])
        w = sum(per["WRITE_SIZE"][k]) / len(per["WRITE_SIZE"][k])
        return {"kernel": k, "dispatches": len(per["FETCH_SIZE"][k]), "fetch_kib_raw": round(f, 1),
                "write_kib_raw": round(w, 1), "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
                "bytes_per_launch": int(round((f * fetch_scale + w * write_scale) * 1024))}

    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    codec = kernel("q8_") is not None
    if workload.startswith("decode_"):  # decode_warm / decode_hbm: the --decode-at-scale-only runs
        cmd = PMC_COMMAND_DECODE.format(ctr="<FETCH_SIZE|WRITE_SIZE>", scale=workload[len("decode_"):])
    else:
        cmd = (PMC_COMMAND_CODEC if codec else PMC_COMMAND).format(ctr="<FETCH_SIZE|WRITE_SIZE>", workload=workload)
    group = "codec" if codec else "scan"
    entry = {"sources": group, "source_hash": kernel_source_hash(group), "command": cmd,
             "copy_calibration": {"kernel": copy_name, "fetch_scale": round(fetch_scale, 4),
                                  "write_scale": round(write_scale, 4)}}
    if codec:
        entry.update({"quantize": kernel("q8_quantize"), "dequant_sum": kernel("q8_dequant_sum")})
        entry["bytes_per_launch"] = entry["quantize"]["bytes_per_launch"] if entry["quantize"] else None
    else:
        entry.update({"prefill": kernel("prefill_"), "decode": kernel("decode_")})
        entry["bytes_per_launch"] = entry["prefill"]["bytes_per_launch"] if entry["prefill"] else None
    if (rec.get(workload) or {}).get("issue"):
        entry["issue"] = rec[workload]["issue"]  # kept: recorded from its own counter run
    rec[workload] = entry
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(entry, indent=1))


def cpu_baseline(w, prm, seq_dev, toks_dev):
    """Time the oracle (fp64, C, all host cores) on the same bits: the full prefill, then the
    decode steps from its own cache."""
    import oracle
    import torch

    cores = oracle.default_threads()
    seq = {k: v.cpu() for k, v in seq_dev.items()}
    t0 = time.perf_counter()
    _, h, c = oracle.prefill(seq, prm, nthreads=cores)
    t1 = time.perf_counter()
    T = len(toks_dev)
    toks = [{k: v.cpu() for k, v in t.items()} for t in toks_dev]
    t2 = time.perf_counter()
    for tok in toks:
        _, h, c = oracle.decode_step(tok, prm, h, c, nthreads=cores)
    t3 = time.perf_counter()
    elems = w.batch * w.seqlen * w.d_inner
    # one core: the same prefill on a 1/cores share of the channels (work is linear in channels)
    sub = max(1, w.d_inner // cores)
    seq1 = {k: (v[:, :sub].contiguous() if k in ("x", "dt", "z") else v) for k, v in seq.items()}
    prm1 = {k: (None if v is None else v[:sub].contiguous()) for k, v in prm.items()}
    t4 = time.perf_counter()
    oracle.prefill(seq1, prm1, nthreads=1)
    t5 = time.perf_counter()
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(elems / (t1 - t0) / 1e9, 4), "unit": "Gelem/s", "cores": cores, "kind": "oracle",
            "sample": f"whole prefill of the workload ({w.batch}x{w.seqlen}x{w.d_inner} elements) on the same bf16 "
                      f"bits, then {T} decode steps from the oracle's own cache; threads over channels",
            "prefill_s": round(t1 - t0, 3), "decode_us_per_step": round((t3 - t2) / max(T, 1) * 1e6, 1),
            "value_1core": round(w.batch * w.seqlen * sub / (t5 - t4) / 1e9, 5),
            "sample_1core": f"{sub} of the {w.d_inner} channels on one thread", "cpu_model": model}


def codec_bytes(n, nb, es, parts):
    """Algorithmic HBM bytes of the codec kernels: quantize reads the io tensor and writes one
    code per element plus one fp32 scale per block; dequant-sum reads every part's codes and
    scales and writes the io tensor."""
    return n * es + n + 4 * nb, parts * (n + 4 * nb) + n * es


def codec_cpu_baseline(xs_dev, block, elems_sample):
    """Time the numpy codec oracle on the host on a bounded sample: the first `elems_sample`
    elements of every part, quantized, then dequantized and summed."""
    import numpy as np
    from oracle import codec as C

    xs = [x[:elems_sample].float().cpu().numpy() for x in xs_dev]
    t0 = time.perf_counter()
    enc = [C.quantize(x, block) for x in xs]
    t1 = time.perf_counter()
    C.dequantize_sum(np.stack([e[0] for e in enc]), np.stack([e[1] for e in enc]), block)
    t2 = time.perf_counter()
    n, nb, P = elems_sample, -(-elems_sample // block), len(xs)
    qb, db = codec_bytes(n, nb, 2, P)
    t_step = (t1 - t0) / P + (t2 - t1)
    return {"value": round((qb + db) / t_step / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {elems_sample} elements of each of the {P} parts: quantize (time per part) plus the "
                      f"{P}-part dequant-sum, numpy on one thread; algorithmic bytes of that sample / time",
            "quantize_s_per_part": round((t1 - t0) / P, 4), "dequant_sum_s": round(t2 - t1, 4)}


def bench_codec(args):
    """One step = quantize this rank's partial + dequantize-and-sum the P parts received."""
    import torch

    import selective_state_space_causal_amd as ssm
    from selective_state_space_causal_amd import inputs as I

    w = I.AGGREGATES[args.codec]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ssm.load()
    n, block, P = w.tokens * w.d_model, w.block, w.parts
    es = 2 if w.io == "bf16" else 4
    nb = ssm.q8_num_blocks(n, block)
    log(f"bench: codec {w.name} tokens={w.tokens} d_model={w.d_model} parts={P} block={block} io={w.io}")
    xs = [I.make_aggregate(w.tokens, w.d_model, w.io, seed=0, part=p, device=dev).reshape(-1) for p in range(P)]
    qs = [torch.empty(n, dtype=torch.int8, device=dev) for _ in range(P)]
    ss = [torch.empty(nb, dtype=torch.float32, device=dev) for _ in range(P)]
    for p in range(P):  # the parts "received" from the other ranks
        ssm.q8_quantize(xs[p], block, q=qs[p], scales=ss[p])
    y = torch.empty(n, dtype=xs[0].dtype, device=dev)
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("bench: copy calibration: 1 GiB read + 1 GiB written")
        del src, dst
    stream = torch.cuda.current_stream()

    def step(e):
        e[0].record(stream)
        ssm.q8_quantize(xs[0], block, q=qs[0], scales=ss[0], stream=stream)
        e[1].record(stream)
        ssm.q8_dequant_sum(qs, ss, block, xs[0].dtype, y=y, stream=stream)
        e[2].record(stream)

    marks, secs = timed_steps(step, 3, args.warmup, args.steps)
    t0, t1 = 0.0, secs
    q_ms = sum(a.elapsed_time(b) for a, b, _ in marks) / len(marks)
    d_ms = sum(b.elapsed_time(c) for _, b, c in marks) / len(marks)
    qb, db = codec_bytes(n, nb, es, P)
    q_gbps, d_gbps = qb / (q_ms * 1e-3) / 1e9, db / (d_ms * 1e-3) / 1e9
    step_gbps = (qb + db) / ((q_ms + d_ms) * 1e-3) / 1e9
    log(f"bench: quantize {q_ms * 1e3:.1f} us ({q_gbps:.0f} GB/s), dequant-sum of {P} parts {d_ms * 1e3:.1f} us "
        f"({d_gbps:.0f} GB/s)")
    rec = {
        "metric": "int8 codec GB/s (quantize one rank's partial + dequant-sum of the parts; algorithmic bytes)",
        "value": round(step_gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "d_model": w.d_model, "parts": P, "block": block,
                   "io": w.io, "parallelism": "none (the collective between ranks is not part of the library)"},
        "quantize": {"us": round(q_ms * 1e3, 2), "algorithmic_bytes": qb, "achieved": round(q_gbps, 1),
                     "frac": round(q_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic_from_profiles(w.name, "quantize")},
        "dequant_sum": {"us": round(d_ms * 1e3, 2), "algorithmic_bytes": db, "achieved": round(d_gbps, 1),
                        "frac": round(d_gbps / HBM_PEAK_GBPS, 4),
                        "traffic": traffic_from_profiles(w.name, "dequant_sum")},
        "roofline": {"kernel": "dequant_sum", "bound": "hbm", "achieved": round(d_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(d_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profiles(w.name, "dequant_sum")},
    }
    if not args.no_cpu_baseline:
        log("bench: timing the codec oracle on the host")
        rec["cpu_baseline"] = codec_cpu_baseline(xs, block, n)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def bench_layer(args):
    """One step = one rank's mixer layer over the prompt: in_proj (x and z), conv front, x_proj
    (low-rank step input, B, C), dt_proj, the scan, out_proj (partial in the io dtype)."""
    import torch

    import selective_state_space_causal_amd as ssm
    from selective_state_space_causal_amd import inputs as I
    from selective_state_space_causal_amd import layer

    w = I.LAYERS[args.layer]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ssm.load()
    B, L, DM, D, R, N = w.batch, w.seqlen, w.d_model, w.d_inner, w.dt_rank, w.d_state
    log(f"bench: layer {w.name} B={B} L={L} d_model={DM} d_inner={D} dt_rank={R} d_state={N} io={w.io}")
    prm = {k: v.to(dev) for k, v in I.make_params(D, N).items() if v is not None}
    wts = I.make_proj_weights(DM, D, R, N, w.io, device=dev)
    hidden = I.make_hidden(B, L, DM, w.io, device=dev)
    pj = ssm.Projector(dev)
    stream = torch.cuda.current_stream()
    bufs = layer.alloc_buffers(hidden, wts, N)
    plan = layer.stages(hidden, wts, prm, pj, bufs, stream)
    names = [n for n, _ in plan]

    def step(evs):
        evs[0].record(stream)
        for i, (_, f) in enumerate(plan):
            f()
            evs[i + 1].record(stream)

    marks, secs = timed_steps(step, len(names) + 1, args.warmup, args.steps)
    t0, t1 = 0.0, secs
    ms = [sum(m[i].elapsed_time(m[i + 1]) for m in marks) / len(marks) for i in range(len(names))]
    total = sum(ms)
    tokens = B * L
    flops = {"in_proj_xz": 4 * tokens * DM * D, "in_proj_x": 2 * tokens * DM * D, "in_proj_z": 2 * tokens * DM * D,
             "x_proj_dt": 2 * tokens * D * R, "conv_xproj": 2 * tokens * D * (R + 2 * N),
             "x_proj_B": 2 * tokens * D * N, "x_proj_C": 2 * tokens * D * N, "dt_proj": 2 * tokens * R * D,
             "out_proj": 2 * tokens * D * DM}
    stages_rec = {}
    for n, t in zip(names, ms):
        e = {"ms": round(t, 4)}
        if n in flops:
            tf = flops[n] / (t * 1e-3) / 1e12
            e.update({"tflops": round(tf, 1), "mfma_frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)})
        stages_rec[n] = e
    log("bench: " + ", ".join(f"{n} {t * 1e3:.1f} us" for n, t in zip(names, ms)) + f"; layer {total:.3f} ms")
    gemm = stages_rec[names[0]]
    rec = {
        "metric": "mixer layer tokens/s (one rank's channel slice: projections, conv front, scan)",
        "value": round(tokens / (total * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (random-init weights)",
        "config": {"workload": w.name, "batch": B, "seqlen": L, "d_model": DM, "d_inner": D, "dt_rank": R,
                   "d_state": N, "io": w.io, "parallelism": "none (one rank's shard; its all-reduces are not built)"},
        "layer_ms": round(total, 4), "stages": stages_rec,
        "roofline": {"kernel": "in_proj GEMM (hipBLASLt)", "bound": "mfma", "achieved": gemm["tflops"],
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": gemm["mfma_frac"], "traffic": None},
        "cpu_baseline": None,
    }
    rec["decode"] = {kind: layer_decode_timing(args, w, wts, prm, pj, bufs["h"], bufs["c"], kind == "fused")
                     for kind in ("unfused", "fused")}
    pj.close()
    if not args.no_cpu_baseline:
        log("bench: timing the layer oracle on the host")
        rec["cpu_baseline"] = layer_cpu_baseline(w, hidden, wts, prm, tokens=1024)
    print(json.dumps(rec), flush=True)


def layer_decode_timing(args, w, wts, prm, pj, h, c, fused, T=64):
    """Decode through one rank's layer: T tokens per batch row from the cache the timed prefill
    left (in_proj, the per-token stages -- separate calls, or ssm_decode_fused -- and out_proj),
    captured in one HIP graph and replayed as a serving loop runs it; HIP events around each
    replay.  Reported per token, with the calls per token and the bytes a token must move at
    least (every weight of the slice once, the cache read and written, the token's io)."""
    import torch

    from selective_state_space_causal_amd import inputs as I
    from selective_state_space_causal_amd import layer

    B, DM, D, R, N = w.batch, w.d_model, w.d_inner, w.dt_rank, w.d_state
    dev = h.device
    hidden = I.make_hidden(B, T, DM, w.io, device=dev)
    toks = [hidden[:, t].contiguous() for t in range(T)]
    bufs = layer.alloc_decode_buffers(toks[0], wts, N, fused)
    plans = [layer.decode_stages(toks[t], wts, prm, pj, h, c, bufs, fused) for t in range(T)]
    stream = torch.cuda.current_stream()

    def loop():
        for plan in plans:
            for _, call in plan:
                call()

    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        loop()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop()
    torch.cuda.synchronize()

    def step(e):
        e[0].record(stream)
        graph.replay()
        e[1].record(stream)

    marks, _ = timed_steps(step, 2, args.warmup, args.steps)
    each = sorted(a.elapsed_time(b) * 1e3 / T for a, b in marks)
    us = sum(each) / len(each)
    es = 2 if w.io == "bf16" else 4
    weight_bytes = (2 * D * DM + (R + 2 * N) * D + D * R + DM * D) * es
    tok_bytes = weight_bytes + B * D * ((N + CONV_W - 1) * 4 * 2 + 3 * es) + B * DM * 2 * es + D * (N + 7) * 4
    gbps = tok_bytes / (us * 1e-6) / 1e9
    names = [n for n, _ in plans[0]]
    log(f"bench: layer decode ({'fused' if fused else 'separate calls'}): {us:.2f} us/token over {len(names)} calls "
        f"({', '.join(names)}), {gbps:.0f} GB/s")
    del graph
    return {"us_per_token": round(us, 3), "us_per_token_range": [round(each[0], 3), round(each[-1], 3)],
            "calls_per_token": len(names), "calls": names, "tokens_per_replay": T, "mode": "hip_graph",
            "algorithmic_bytes_per_token": tok_bytes, "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4)}


def layer_cpu_baseline(w, hidden, wts, prm, tokens):
    """The oracle's layer (numpy fp64 projections, the C scan on all host cores) on the first
    `tokens` tokens of batch row 0."""
    import oracle
    from oracle import proj as P

    h = hidden[:1, :tokens].cpu()
    wc = {k: v.cpu() for k, v in wts.items()}
    pc = {k: v.cpu() for k, v in prm.items()}
    cores = oracle.default_threads()
    t0 = time.perf_counter()
    P.layer_prefill(h, wc, pc, w.io, nthreads=cores)
    dt = time.perf_counter() - t0
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {tokens} tokens of the layer (batch row 0): numpy fp64 projections (one thread) and the "
                      f"C fp64 scan over {cores} threads", "seconds": round(dt, 3)}


def plain_copy_gbps():
    """Context for the HBM fractions: a plain 1 GiB device copy, timed (it is also the
    byte-counter calibration dispatch of the rocprofv3 --pmc runs)."""
    import torch

    stream = torch.cuda.current_stream()
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = TimingEvent(), TimingEvent()
    c0.record(stream)
    dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    gbps = 2 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    log(f"bench: plain 1 GiB copy: {gbps:.0f} GB/s (read + write)")
    return gbps


# The decode step where it moves enough bytes per step to be bound by memory rather than by
# launch latency, on two caches of the Mamba-2.8B layer shape (d_inner 5120, d_state 16):
#   warm: batch 64, the mamba2.8b workload's cache (21 MB of h + 3.9 MB of conv window), which
#         stays in the 256 MB last-level cache (Infinity Cache) across a replay;
#   hbm:  batch 1024 (336 MB of h + 63 MB of conv window), larger than that cache, so that
#         every step streams its cache from HBM.
DECODE_SCALES = {"warm": (64, 256), "hbm": (1024, 64)}  # batch, steps per replay
LLC_BYTES = 256 << 20


def decode_at_scale(args, copy_gbps, scale="warm"):
    """The decode step on a cache left by a 64-token prefill of the layer shape, then its
    decode steps on their own seeded tokens, replayed from one captured HIP graph per step
    sequence as a serving loop runs them.  Inputs resident in HBM before timing; HIP events
    around each replay."""
    import torch

    import selective_state_space_causal_amd as ssm
    from selective_state_space_causal_amd import inputs as I

    w = I.WORKLOADS["mamba2.8b"]
    B, T = DECODE_SCALES[scale]
    D, N = w.d_inner, w.d_state
    es = 2 if w.io == "bf16" else 4
    dev = torch.device("cuda:0")
    prm = I.make_params(D, N, dt_range=w.dt_range)
    pd = {k: v.to(dev) for k, v in prm.items()}
    pre = I.make_sequence_device(B, 64, D, N, w.io, stream="prefill", device=dev)
    _, h, c = ssm.prefill(pre["x"], pre["dt"], pre["z"], pre["Bm"], pre["Cm"], pd)
    del pre
    tk = I.make_sequence_device(B, T, D, N, w.io, stream="decode_at_scale", device=dev)
    xs, dts, zs = (tk[k].permute(2, 0, 1).contiguous() for k in ("x", "dt", "z"))  # [T, B, D]
    Bs, Cs = (tk[k].permute(1, 0, 2).contiguous() for k in ("Bm", "Cm"))          # [T, B, N]
    del tk
    ys = torch.empty_like(xs)
    stream = torch.cuda.current_stream()

    def loop():
        for t in range(T):
            ssm.decode_step(xs[t], dts[t], zs[t], Bs[t], Cs[t], pd, h, c, y_t=ys[t])

    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        loop()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop()
    torch.cuda.synchronize()

    def step(e):
        e[0].record(stream)
        graph.replay()
        e[1].record(stream)

    marks, _ = timed_steps(step, 2, args.warmup, args.steps)
    each = sorted(a.elapsed_time(b) * 1e3 / T for a, b in marks)
    us = sum(each) / len(each)
    dbytes = decode_bytes(B, D, N, es)
    gbps = dbytes / (us * 1e-6) / 1e9
    cache_bytes = B * D * (N + CONV_W - 1) * 4
    log(f"bench: decode at scale ({scale}: batch {B}, {cache_bytes / 2**20:.0f} MiB of cache, {T} steps per "
        f"replay): {us:.2f} us/step, {gbps:.0f} GB/s")
    del graph
    return {"workload": "mamba2.8b-shaped cache" if B != w.batch else "mamba2.8b", "batch": B, "d_inner": D,
            "d_state": N, "steps_per_replay": T, "cache_bytes": cache_bytes,
            "cache_resident_in_llc": cache_bytes < LLC_BYTES,
            "state_from": "64-token prefill of the same shape", "mode": "hip_graph",
            "us_per_step": round(us, 3), "us_per_step_range": [round(each[0], 3), round(each[-1], 3)],
            "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4), "frac_of_copy": round(gbps / copy_gbps, 4),
            "algorithmic_bytes": dbytes}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="slice7b")
    ap.add_argument("--decode-steps", type=int, default=None, help="override the workload's decode step count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-at-scale", action="store_true",
                    help="skip the decode step timed on the mamba2.8b cache (also skipped with --decode-steps)")
    ap.add_argument("--eager-decode", action="store_true", help="time decode as one host call per step "
                    "instead of replaying the captured HIP graph")
    ap.add_argument("--chunk-hint", type=int, default=0, help="prefill decomposition (0 auto, 1 sequential, 8 windowed)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for scaling rocprofv3 byte counters; the scan "
                         "bench always times one)")
    ap.add_argument("--cold", action="store_true",
                    help="write a 1 GiB scrub buffer (4x the last-level cache) before each timed prefill")
    ap.add_argument("--pool", action="store_true",
                    help="serving form: ragged prompt lengths (uniform in [L/2, L]) and a cache pool of 2*batch "
                         "entries addressed through a random slot map (ssm_prefill_pool / ssm_decode_step_pool)")
    ap.add_argument("--codec", metavar="AGGREGATE", default=None,
                    help="instead of the scan, time the int8 codec on an aggregation-tensor workload "
                         "(tp_prefill_7b or tp_decode_2.8b) and print its own JSON line")
    ap.add_argument("--layer", metavar="LAYER", default=None,
                    help="instead of the scan alone, time one rank's mixer layer (layer7b): projections, conv "
                         "front, scan, and print its own JSON line")
    ap.add_argument("--decode-at-scale-only", choices=sorted(DECODE_SCALES), default=None,
                    help="time only the decode step on one of the two Mamba-2.8B-shaped caches (warm: batch 64, "
                         "inside the last-level cache; hbm: batch 1024, larger than it) and print its JSON; "
                         "for counter runs")
    ap.add_argument("--record-traffic", metavar="PMC_DIR", default=None,
                    help="write profiles/traffic.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE CSVs and exit")
    ap.add_argument("--record-issue", metavar="CSV", default=None,
                    help="add the prefill kernel's VALU issue occupancy to profiles/traffic.json from a rocprofv3 "
                         "--pmc counter_collection.csv with SQ_WAVES, SQ_WAVE_CYCLES, SQ_ACTIVE_INST_VALU, and exit")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.record_traffic, args.codec or args.workload)
        return
    if args.record_issue:
        record_issue(args.record_issue, args.workload)
        return

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the channel-local recurrence would shard by channel with no exchange inside it).",
              file=sys.stderr)
        sys.exit(2)

    if args.decode_at_scale_only:
        import torch

        torch.cuda.set_device(0)
        print(json.dumps(decode_at_scale(args, plain_copy_gbps(), args.decode_at_scale_only)), flush=True)
        return
    if args.codec:
        bench_codec(args)
        return
    if args.layer:
        bench_layer(args)
        return

    import torch

    import selective_state_space_causal_amd as ssm
    from selective_state_space_causal_amd import inputs as I

    w = I.WORKLOADS[args.workload]
    T = w.decode_steps if args.decode_steps is None else args.decode_steps
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ssm.load()
    B, L, D, N = w.batch, w.seqlen, w.d_inner, w.d_state
    es = 2 if w.io == "bf16" else 4
    log(f"bench: {w.name} B={B} L={L} D={D} N={N} io={w.io} decode_steps={T}")

    prm = I.make_params(D, N, dt_range=w.dt_range)
    pd = {k: v.to(dev) for k, v in prm.items()}
    seq = I.make_sequence_device(B, L, D, N, w.io, device=dev)
    toks = [{k: v.to(dev) for k, v in I.make_decode_token(B, D, N, t, w.io).items()} for t in range(T)]
    y = torch.empty_like(seq["x"])
    h = torch.empty(B, D, N, dtype=torch.float32, device=dev)
    c = torch.empty(B, D, CONV_W - 1, dtype=torch.float32, device=dev)
    ys = torch.empty(max(T, 1), B, D, dtype=seq["x"].dtype, device=dev)
    nws = ssm.workspace_bytes(B, L, D, N, seq["x"].dtype)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev) if nws else None

    stream = torch.cuda.current_stream()
    ev = TimingEvent
    copy_gbps = plain_copy_gbps()
    scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev) if args.cold else None
    elems = B * L * D
    if args.pool:
        g = torch.Generator().manual_seed(1)
        lens = torch.randint(L // 2, L + 1, (B,), generator=g, dtype=torch.int32)
        lens[0] = L
        pool = 2 * B
        slots = torch.randperm(pool, generator=g)[:B].to(torch.int32)
        elems = int(lens.sum()) * D
        lens_d, slots_d = lens.to(dev), slots.to(dev)
        hp = torch.zeros(pool, D, N, dtype=torch.float32, device=dev)
        cp = torch.zeros(pool, D, CONV_W - 1, dtype=torch.float32, device=dev)
        log(f"bench: pool form: {pool} cache entries, lengths {int(lens.min())}..{int(lens.max())}")

    def decode_one(t, s=None):
        tk = toks[t]
        if args.pool:
            ssm.decode_step_pool(tk["x"], tk["dt"], tk["z"], tk["Bm"], tk["Cm"], pd, slots_d, hp, cp,
                                 y_t=ys[t], stream=s)
        else:
            ssm.decode_step(tk["x"], tk["dt"], tk["z"], tk["Bm"], tk["Cm"], pd, h, c, y_t=ys[t], stream=s)

    def decode_loop(s=None):
        for t in range(T):
            decode_one(t, s)

    # The decode loop as a serving loop runs it: captured once in a HIP graph, replayed per
    # request.  (An eager, one-launch-per-call loop is timed separately below.)
    graph = None
    if T and not args.eager_decode:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            decode_loop()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode_loop()
        torch.cuda.synchronize()

    def step(e):
        e0, e1, e2 = e
        if scrub is not None:  # cold: 1 GiB written (4x the last-level cache) before the timed region
            scrub.fill_(0.0)
        e0.record(stream)
        if args.pool:
            ssm.prefill_pool(seq["x"], seq["dt"], seq["z"], seq["Bm"], seq["Cm"], pd, slots_d, hp, cp,
                             seqlens=lens_d, y=y, stream=stream, chunk_hint=args.chunk_hint)
        else:
            ssm.prefill(seq["x"], seq["dt"], seq["z"], seq["Bm"], seq["Cm"], pd, y=y, h_out=h, conv_out=c,
                        workspace=ws, stream=stream, chunk_hint=args.chunk_hint)
        e1.record(stream)
        if graph is not None:
            graph.replay()
        else:
            decode_loop(stream)
        e2.record(stream)

    marks, secs = timed_steps(step, 3, args.warmup, args.steps)
    t0, t1 = 0.0, secs

    eager_us = None
    if T:  # eager decode loop (one host call per step), for reference
        e0, e1 = ev(), ev()
        decode_loop(stream)
        torch.cuda.synchronize()
        e0.record(stream)
        decode_loop(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / T

    cold_first_us = None
    if T:  # one decode step with every cache scrubbed first: the first token after an idle spell
        scrub_c = scrub if scrub is not None else torch.empty(1 << 28, dtype=torch.float32, device=dev)
        scrub_c.fill_(0.0)
        e0, e1 = ev(), ev()
        e0.record(stream)
        decode_one(0, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        cold_first_us = e0.elapsed_time(e1) * 1e3
        del scrub_c

    pre_each = sorted(a.elapsed_time(b) for a, b, _ in marks)
    dec_each = sorted(b.elapsed_time(c_) for _, b, c_ in marks)
    pre_ms = sum(pre_each) / len(pre_each)
    dec_ms = sum(dec_each) / len(dec_each)
    median = lambda v: 0.5 * (v[(len(v) - 1) // 2] + v[len(v) // 2])
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gelem = elems / (pre_ms * 1e-3) / 1e9
    pbytes = prefill_bytes(B, L, D, N, es)
    if args.pool:  # only the real tokens of each row move
        ntok = elems // D
        pbytes = ntok * D * 4 * es + ntok * 2 * N * es + B * D * (N + CONV_W - 1) * 4 + D * (N + 7) * 4
    dbytes = decode_bytes(B, D, N, es)
    p_gbps = pbytes / (pre_ms * 1e-3) / 1e9
    d_us = dec_ms * 1e3 / T if T else None
    d_gbps = dbytes / (d_us * 1e-6) / 1e9 if T else None
    traffic = traffic_from_profiles(w.name)
    log(f"bench: prefill {pre_ms:.3f} ms ({gelem:.1f} Gelem/s, {p_gbps:.0f} GB/s)" +
        (f", decode {d_us:.2f} us/step ({'graph' if graph is not None else 'eager'}; eager {eager_us:.2f} us/step)"
         if T else ""))

    rec = {
        "metric": "prefill Gelem/s (B·L·d_inner) + decode µs/step; % of HBM peak",
        "value": round(gelem, 3), "unit": "Gelem/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name + ("+pool" if args.pool else ""), "batch": B, "seqlen": L, "d_inner": D,
                   "d_state": N, "d_conv": CONV_W, "io": w.io, "state": "f32", "decode_steps": T,
                   "parallelism": "none (one GPU's channel slice)",
                   "tokens": elems // D, "pool_entries": 2 * B if args.pool else None},
        "prefill_ms": round(pre_ms, 4),
        "prefill_ms_median": round(median(pre_each), 4),
        "prefill_ms_range": [round(pre_each[0], 4), round(pre_each[-1], 4)],
        "decode_us_per_step": None if d_us is None else round(d_us, 3),
        "decode_us_per_step_median": None if not T else round(median(dec_each) * 1e3 / T, 3),
        "decode_mode": "hip_graph" if graph is not None else "eager",
        "decode_us_per_step_eager": None if eager_us is None else round(eager_us, 3),
        "decode_us_cold_first_step": None if cold_first_us is None else round(cold_first_us, 3),
        "prefill_hbm": {"achieved": round(p_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(p_gbps / HBM_PEAK_GBPS, 4), "frac_of_copy": round(p_gbps / copy_gbps, 4),
                        "algorithmic_bytes": pbytes},
        "decode_hbm": None if not T else {"achieved": round(d_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                          "frac": round(d_gbps / HBM_PEAK_GBPS, 4),
                                          "frac_of_copy": round(d_gbps / copy_gbps, 4), "algorithmic_bytes": dbytes},
        "copy_gbps": round(copy_gbps, 1),
        "cache_state": "cold (1 GiB scrub before each prefill)" if args.cold else "warm",
        "cache_benefit": None if not T else round(pre_ms * 1e3 / d_us, 1),
        "roofline": dict(kernel="prefill", **valu_roofline(issue_from_profiles(w.name), calib_from_profiles(), pre_ms),
                         traffic=traffic, hbm_frac=round(p_gbps / HBM_PEAK_GBPS, 4),
                         flops_per_element=flops_per_element(N),
                         fp32_tflops=round(flops_per_element(N) * elems / (pre_ms * 1e-3) / 1e12, 3)),
    }
    # With the decode measurement only (not on prefill-only workloads), not in the pool form, not
    # on mamba2.8b itself (its line is that measurement), not when the decode step count is
    # overridden (the counter runs) and not when asked not to.
    if T and not (args.pool or w.name == "mamba2.8b" or args.decode_steps is not None or args.no_decode_at_scale):
        rec["decode_at_scale"] = decode_at_scale(args, copy_gbps, "warm")
        rec["decode_at_scale_hbm"] = decode_at_scale(args, copy_gbps, "hbm")
    if args.pool and not args.no_cpu_baseline:
        log("bench: the CPU baseline is defined on the full workload; skipped in the pool form")
        args.no_cpu_baseline = True
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host cores")
        rec["cpu_baseline"] = cpu_baseline(w, prm, seq, toks)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
