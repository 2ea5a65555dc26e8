"""Summarise the parity margins the GPU tests recorded (tests/gpu_common.py: run the GPU tests
with SSM_PARITY_MARGINS=<file>.json) as a markdown table.

    python -m tests.parity_margins <margins.json> [command that produced it]

For each test: the largest |gpu - ref| / (1 + |ref|) seen on y and on h, as a fraction of the
tolerance tau each comparison used; for the full-size decode runs, the per-step series of the
same quantity, condensed to its largest value and its value over the first and last eighth of
the steps (a growing error would show there)."""
from __future__ import annotations

import json
import sys


def fmt(v, tau):
    return f"{v:.2e} ({v / tau:.3f} tau)"


def summarise(path, command=None):
    d = json.load(open(path))
    tests = d["tests"]
    out = ["# Parity margins of the GPU tests", ""]
    if command:
        out += ["Produced by:", "", "```", command, "```", ""]
    out += [f"{len(tests)} tests recorded a comparison (pytest exit status {d.get('exitstatus')}). "
            "Error = max |gpu - ref| / (1 + |ref|) over every compared element; tau = 1e-4 for fp32 io, "
            "2e-2 for bf16 io. Conv caches are compared bit for bit and do not appear here.", ""]
    out += ["bf16 io tests are also held to a tighter bar (tests/gpu_common.py `tight_ratio`, asserted): h within "
            "the fp32 bar 1e-4 (1 + |ref|), y within half a bf16 ulp (2^-8 |ref|) plus twice the fp32 bar; the "
            "`tight` columns give the largest share of that bar used.", ""]
    out += ["| Test | y | h | tau | y tight | h tight |", "|---|---|---|---|---|---|"]
    worst, worst_t = {}, {}
    for name in sorted(tests):
        rec = tests[name]
        tau = next((v["tau"] for k, v in rec.items() if k != "per_step"), None)
        y = rec.get("y", {}).get("err")
        h = rec.get("h", {}).get("err")
        short = name.split("::", 1)[-1]
        yt = rec.get("y", {}).get("tight")
        ht = rec.get("h", {}).get("tight")
        out.append(f"| `{short}` | {fmt(y, tau) if y is not None else '-'} | {fmt(h, tau) if h is not None else '-'} "
                   f"| {tau:g} | {'-' if yt is None else f'{yt:.3f}'} | {'-' if ht is None else f'{ht:.3f}'} |")
        for k in ("y", "h"):
            if k in rec:
                r = rec[k]["err"] / rec[k]["tau"]
                if r > worst.get(k, (0, ""))[0]:
                    worst[k] = (r, short)
                t = rec[k].get("tight")
                if t is not None and t > worst_t.get(k, (0, ""))[0]:
                    worst_t[k] = (t, short)
    out += [""]
    for k, (r, n) in sorted(worst.items()):
        out.append(f"Largest {k} margin: {r:.3f} tau (`{n}`).")
    for k, (r, n) in sorted(worst_t.items()):
        out.append(f"Largest share of the tight bf16 bar on {k}: {r:.3f} (`{n}`).")
    series = [(n, r["per_step"]) for n, r in sorted(tests.items()) if "per_step" in r]
    if series:
        out += ["", "## Decode steps at full size (per-step largest error over the sampled channels)", "",
                "| Test | output | steps | max | first eighth (max) | last eighth (max) |", "|---|---|---|---|---|---|"]
        for name, per in series:
            tau = next(v["tau"] for k, v in tests[name].items() if k != "per_step")
            for k, s in sorted(per.items()):
                e = max(1, len(s) // 8)
                out.append(f"| `{name.split('::', 1)[-1]}` | {k} | {len(s)} | {fmt(max(s), tau)} | "
                           f"{max(s[:e]):.2e} | {max(s[-e:]):.2e} |")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    sys.stdout.write(summarise(sys.argv[1], " ".join(sys.argv[2:]) or None))
