"""Per-kernel summaries of rocprofv3 counter collections.

A counter pass is one run of the bench under rocprofv3 with one group of
counters (the hardware collects a few per block at a time), e.g.

    rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU ... GRBM_GUI_ACTIVE --output-format csv \
        -d /tmp/pmc_a -o run -- python3 bench.py --steps 3 --warmup 2 --no-cpu-baseline

Then, per pass, ``collect`` reduces the per-dispatch CSV rows to one record
per (kernel, grid size): the number of dispatches and the mean of every
counter per dispatch (rocprofv3 sums each counter over its hardware
instances: SQ counters over every CU's sequencer, GRBM_GUI_ACTIVE over the
eight XCDs); ``table`` merges passes and prints the derived figures as a
markdown table:

    python -m paged_hybrid_kv_amd.counters collect /tmp/pmc_a pass_a.json
    python -m paged_hybrid_kv_amd.counters table pass_a.json pass_b.json ... [--match substr ...]

and, for a kernel-trace run (rocprofv3 --kernel-trace --stats --output-format csv
-d DIR ...), ``trace`` prints calls and mean / min / max duration per (kernel,
grid size), which separates the launches of one kernel at different shapes:

    python -m paged_hybrid_kv_amd.counters trace DIR [--match substr ...]

Derived figures (per dispatch):
  cycles        GRBM_GUI_ACTIVE / 8 (the eight XCDs run the dispatch side by side)
  VALU, MFMA, LDS, VMEM, SALU instr/wave   SQ_INSTS_* / SQ_WAVES
  VALU active   SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES (share of a wave's lifetime issuing VALU)
  MFMA busy     SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)
  LDS active    SQ_ACTIVE_INST_LDS / SQ_WAVE_CYCLES
  bank conflict SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS
  LDS wait      SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES
  any wait      SQ_WAIT_ANY / SQ_WAVE_CYCLES
  FETCH, WRITE  FETCH_SIZE, WRITE_SIZE in KiB (raw; the bench's --copy-calib copies give the scale)
"""

from __future__ import annotations

import csv
import glob
import json
import os
import re
import sys

SIMDS = 1024
XCDS = 8


def _kernel_name(raw: str) -> str:
    name = raw.replace("void ", "").replace("(anonymous namespace)::", "").replace("gw::", "")
    return re.sub(r"\(.*", "", name).strip()


def collect(run_dir: str) -> dict:
    """{"kernel grid=N": {"dispatches", "mean": {counter: mean per dispatch}}} over every
    counter_collection.csv under run_dir."""
    out = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        disp = {}
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (r["Dispatch_Id"], _kernel_name(r["Kernel_Name"]), r["Grid_Size"])
                d = disp.setdefault(key, {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for (_, name, grid), cs in disp.items():
            e = out.setdefault(f"{name} grid={grid}", {"dispatches": 0, "sum": {}})
            e["dispatches"] += 1
            for c, v in cs.items():
                e["sum"][c] = e["sum"].get(c, 0.0) + v
    return {k: {"dispatches": e["dispatches"], "mean": {c: v / e["dispatches"] for c, v in sorted(e["sum"].items())}}
            for k, e in out.items()}


def _ratio(m, a, b, scale=1.0):
    if a in m and b in m and m[b]:
        return m[a] / (m[b] * scale)
    return None


def derived(m: dict) -> dict:
    cyc = m["GRBM_GUI_ACTIVE"] / XCDS if "GRBM_GUI_ACTIVE" in m else None
    d = {"cycles": cyc}
    for k, c in (("VALU/wave", "SQ_INSTS_VALU"), ("MFMA/wave", "SQ_INSTS_MFMA"), ("LDS/wave", "SQ_INSTS_LDS"),
                 ("VMEM/wave", "SQ_INSTS_VMEM"), ("SALU/wave", "SQ_INSTS_SALU")):
        d[k] = _ratio(m, c, "SQ_WAVES")
    d["VALU active"] = _ratio(m, "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES")
    d["MFMA busy"] = (m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS)
                      if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in m else None)
    d["LDS active"] = _ratio(m, "SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES")
    d["bank conflict"] = _ratio(m, "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS")
    d["LDS wait"] = _ratio(m, "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES")
    d["any wait"] = _ratio(m, "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")
    d["FETCH KiB"] = m.get("FETCH_SIZE")
    d["WRITE KiB"] = m.get("WRITE_SIZE")
    return d


def _fmt(k, v):
    if v is None:
        return "-"
    if k in ("VALU active", "MFMA busy", "LDS active", "bank conflict", "LDS wait", "any wait"):
        return f"{100 * v:.1f}%"
    if k in ("cycles", "FETCH KiB", "WRITE KiB"):
        return f"{v:,.0f}"
    return f"{v:.1f}"


def table(passes: list[dict], match: list[str] | None = None) -> str:
    merged = {}
    for p in passes:
        for k, e in p.items():
            r = merged.setdefault(k, {"dispatches": e["dispatches"], "mean": {}})
            r["mean"].update(e["mean"])
    cols = ["cycles", "VALU/wave", "MFMA/wave", "LDS/wave", "VMEM/wave", "SALU/wave", "VALU active", "MFMA busy",
            "LDS active", "bank conflict", "LDS wait", "any wait", "FETCH KiB", "WRITE KiB"]
    lines = ["| kernel (grid) | dispatches | " + " | ".join(cols) + " |", "|---" * (len(cols) + 2) + "|"]
    for k in sorted(merged):
        if match and not any(s in k for s in match):
            continue
        e = merged[k]
        d = derived(e["mean"])
        lines.append(f"| `{k}` | {e['dispatches']} | " + " | ".join(_fmt(c, d[c]) for c in cols) + " |")
    return "\n".join(lines)


def trace(run_dir: str, match: list[str] | None = None) -> str:
    per = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = _kernel_name(r["Kernel_Name"])
                grid = r.get("Grid_Size") or r.get("Grid_Size_X", "")
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
                per.setdefault(f"{name} grid={grid}", []).append(dur)
    lines = ["| kernel (grid) | calls | mean us | min us | max us |", "|---|---|---|---|---|"]
    for k in sorted(per):
        if match and not any(s in k for s in match):
            continue
        v = per[k]
        lines.append(f"| `{k}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(lines)


def main(argv):
    if len(argv) >= 3 and argv[0] == "collect":
        res = collect(argv[1])
        with open(argv[2], "w") as f:
            json.dump(res, f, indent=1)
        print(f"{len(res)} kernel/grid entries -> {argv[2]}")
        return 0
    if len(argv) >= 2 and argv[0] == "trace":
        match = [argv[i + 1] for i, a in enumerate(argv) if a == "--match" and i + 1 < len(argv)]
        print(trace(argv[1], match or None))
        return 0
    if len(argv) >= 2 and argv[0] == "table":
        files, match = [], []
        it = iter(argv[1:])
        for a in it:
            if a == "--match":
                match.append(next(it))
            else:
                files.append(a)
        print(table([json.load(open(f)) for f in files], match or None))
        return 0
    print(__doc__)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
