"""Per-workgroup timeline of the decode kernels, from the trace build.

The trace build (``python -m paged_hybrid_kv_amd.build --trace`` writes
libgw_trace.so: the same sources compiled with GW_TRACE) has the local and
global decode kernels record event times per workgroup (the 100 MHz
constant clock) into a device buffer; the slots are listed in the kernels.
This module runs layers of the hybrid decode step (and, with --big, the
global family at 8 x 131072 tokens) through that build and prints, per
kernel, where a workgroup's time goes: start-up until its first pages are
in, the page loop per unit of work, the tail after the loop, and the spread
of workgroup starts and ends across the launch.

    python -m paged_hybrid_kv_amd.trace [--big] [--prefill] [--dump rows.npz]

With --prefill it times the prompt-row kernels instead, in one local and
one global layer of the mixed step (4 new 512-token prompts) and of the
chunked-prefill step (a 512-token chunk after a 3584-token prefix): per
workgroup, the start-up until the first step's keys are in LDS, the cost of
a step of the key loop (fitted over workgroups with different range
lengths), the write-out, and when the workgroups start and end.

It needs the GPU and the trace build; it changes nothing in the product
library (libgw.so), which records nothing.
"""

from __future__ import annotations

import ctypes
import os
import sys

import numpy as np

from . import build as B
from . import gw

SLOTS = 16
TICK_US = 0.01   # s_memrealtime runs at 100 MHz


def load_trace_lib():
    if not os.path.exists(B.TRACE_LIB):
        raise RuntimeError(f"{B.TRACE_LIB} is missing: build it with python -m paged_hybrid_kv_amd.build --trace")
    if gw._lib is not None and gw.LIB_PATH != B.TRACE_LIB:
        raise RuntimeError("the product library is already loaded in this process")
    gw.LIB_PATH = B.TRACE_LIB
    L = gw.lib()
    L.gw_trace_buffer.restype = ctypes.c_int
    L.gw_trace_buffer.argtypes = [ctypes.c_void_p]
    return L


def _med(x):
    return float(np.median(x)) if len(x) else float("nan")


def summarize(name: str, rows: np.ndarray, unit_slot: int, unit_name: str, loop_start: int, loop_end: int) -> str:
    """rows: [workgroups][16] of one launch; rows of workgroups that did no work are zero in slot 3."""
    a = rows[rows[:, 3] != 0]
    t0 = rows[rows[:, 2] != 0, 2].min()
    us = lambda x: (x.astype(np.int64) - int(t0)) * TICK_US
    units = (a[:, 1] & 0xffff).astype(np.int64)
    xcc = (a[:, 0] & 0xf).astype(np.int64)
    startup = (a[:, 3] - a[:, 2]) * TICK_US
    loop = (a[:, loop_end].astype(np.int64) - a[:, loop_start].astype(np.int64)) * TICK_US
    per_unit = loop / np.maximum(units, 1)
    tail = (a[:, 7].astype(np.int64) - a[:, loop_end].astype(np.int64)) * TICK_US
    end = us(a[:, 7])
    out = [f"| {name} | {len(a)} | {_med(units):.0f} | {us(a[:, 2]).max():.2f} | {_med(startup):.2f} | "
           f"{_med(per_unit):.3f} | {_med(loop):.2f} | {_med(tail):.2f} | {_med(end):.2f} | {end.max():.2f} | "
           + " ".join(f"{end[xcc == x].max():.1f}" if (xcc == x).any() else "-" for x in range(8)) + " |"]
    return "\n".join(out)


HEADER = ("| launch | active WGs | units/WG (med) | last WG start (µs) | start-up: entry → slot 3 (med µs) | "
          "loop per unit (med µs) | loop (med µs) | tail: loop end → exit (med µs) | exit (med µs) | "
          "last exit (µs) | last exit per XCD 0..7 (µs) |\n|---|---|---|---|---|---|---|---|---|---|---|")


PREFILL_HEADER = ("| launch | active WGs | steps/WG min / med / max | last WG start (µs) | start-up: entry → slot 3 "
                  "(med µs) | µs per step (fit) | fixed µs (fit) | middle steps (med µs/step) | wave spread at loop "
                  "end (med µs) | write-out: loop end → exit (med µs) | exit (med µs) | last exit (µs) |\n"
                  "|---|---|---|---|---|---|---|---|---|---|---|---|")


def summarize_prefill(name: str, rows: np.ndarray) -> str:
    """rows: the prompt-row kernel's trace rows (from kTracePrefillRow) of one launch."""
    rows = rows.astype(np.int64)
    a = rows[rows[:, 3] != 0]
    t0 = rows[rows[:, 2] != 0, 2].min()
    us = lambda x: (x - t0) * TICK_US
    n = a[:, 1]
    startup = (a[:, 3] - a[:, 2]) * TICK_US
    loop = (a[:, 4] - a[:, 3]) * TICK_US
    wall = (a[:, 4] - a[:, 2]) * TICK_US
    slope, icpt = np.polyfit(n, wall, 1) if len(np.unique(n)) > 1 else (float("nan"), float("nan"))
    mid = a[n >= 3]
    mid_step = (mid[:, 6] - mid[:, 5]) * TICK_US / np.maximum(mid[:, 1] - 2, 1)
    wend = a[:, 8:16]
    spread = (wend.max(1) - wend[:, :8].min(1)) * TICK_US
    tail = (a[:, 7] - a[:, 4]) * TICK_US
    end = us(a[:, 7])
    return (f"| {name} | {len(a)} | {n.min()} / {_med(n):.0f} / {n.max()} | {us(a[:, 2]).max():.2f} | "
            f"{_med(startup):.2f} | {slope:.3f} | {icpt:.2f} | {_med(mid_step):.3f} | {_med(spread):.2f} | "
            f"{_med(tail):.2f} | {_med(end):.2f} | {end.max():.2f} |")


def run_prefill(dump: str | None = None) -> str:
    import torch

    L = load_trace_lib()
    from .step import HybridStep
    from .synth import HybridShape

    buf = torch.zeros(SLOTS * 8192, dtype=torch.int64, device="cuda")
    raw = {}
    assert L.gw_trace_buffer(buf.data_ptr()) == 0
    lines = ["Per-workgroup event times of the prompt-row kernels, one launch each (trace build), times from "
             "the launch's first workgroup start.  A step is 32 tokens (two pages, local) or one page (global); "
             "the per-step cost and the fixed cost are the least-squares line of entry-to-loop-end time against "
             "the workgroup's step count; middle steps = iteration 1 to the last iteration's start.", "",
             PREFILL_HEADER]
    for prefix, label in ((0, "mixed step"), (3584, "chunked-prefill step")):
        st = HybridStep(shape=HybridShape(prompt_prefix=prefix), with_prompts=True)
        for _ in range(2):
            st.run()
        torch.cuda.synchronize()
        loc = next(x for x in st.layers if x["local"])
        glb = next(x for x in st.layers if not x["local"])
        for kind, x in (("local", loc), ("global", glb)):
            buf.zero_()
            st.attend(x, append=True)
            torch.cuda.synchronize()
            rows = buf.view(-1, SLOTS).cpu().numpy().astype(np.uint64)[4096:]
            raw[f"{kind}_prefill_{prefix}"] = rows
            lines.append(summarize_prefill(f"{label}, layer {x['index']} {kind} prompt rows", rows))
        del st
        torch.cuda.empty_cache()
    L.gw_trace_buffer(None)
    if dump:
        np.savez(dump, **raw)
    return "\n".join(lines)


def run(big: bool = False, layers: int = 4, dump: str | None = None) -> str:
    import torch

    L = load_trace_lib()
    from .step import HybridStep

    buf = torch.zeros(SLOTS * 8192, dtype=torch.int64, device="cuda")
    raw = {}
    assert L.gw_trace_buffer(buf.data_ptr()) == 0
    lines = ["Per-workgroup event times of one launch each (trace build), times from the launch's first "
             "workgroup start.  Local decode: units = virtual pages of wave 0, slot 3 = q and page table in LDS, "
             "loop = slot 3 to wave 0's last page, tail = LDS merge of the waves, partial publish and (last "
             "workgroup of a pair) the split merge.  Global decode: units = page pairs, slot 3 = pair 0 in LDS, "
             "loop = step 1 open to the value waves' loop end (value waves see pair j at step j + 1), tail = "
             "partial or output writes.", "", HEADER]
    st = HybridStep(with_prompts=False)
    loc = [x for x in st.layers if x["local"]]
    glb = [x for x in st.layers if not x["local"]]
    for _ in range(2):
        for x in st.layers:
            st.attend(x, append=True)
    torch.cuda.synchronize()
    for i in range(layers):
        for kind, x in (("local", loc[i]), ("global", glb[i])):
            buf.zero_()
            st.attend(x, append=True)
            torch.cuda.synchronize()
            rows = buf.view(-1, SLOTS).cpu().numpy().astype(np.uint64)
            raw[f"{kind}_{x['index']}"] = rows
            if kind == "local":
                lines.append(summarize(f"step layer {x['index']} local (bf16, 16 slots)", rows, 1, "pages", 3, 4))
            else:
                lines.append(summarize(f"step layer {x['index']} global decode (bf16 compressed)", rows, 1, "pairs",
                                       4, 5))
    del st
    torch.cuda.empty_cache()
    if big:
        from . import runtime as RT, synth as SY
        for fam, fp8, label in ((gw.GW_FAMILY_GLOBAL_COMPRESSED, False, "bf16 compressed"),
                                (gw.GW_FAMILY_GLOBAL_COMPRESSED, True, "e4m3 compressed")):
            rng = np.random.default_rng(3)
            lens = np.full(8, 131072)
            seqs = SY.make_page_table(rng, lens)
            pool = RT.Pool(fam, gw.GW_KV_E4M3 if fp8 else gw.GW_KV_BF16, seqs.num_pages, 1, 128, "cuda")
            pt, stride = RT.i32_dev(seqs.page_table), seqs.page_table.shape[1]
            cos, sin = RT.rope_tables(131072, 128, 512, RT.GLOBAL_THETA)
            g = torch.Generator(device="cuda")
            g.manual_seed(3000)
            for s in range(8):
                for c0 in range(0, 131072, 32768):
                    v = torch.randn(32768, 512, device="cuda", generator=g).to(torch.bfloat16)
                    si = torch.full((32768,), s, dtype=torch.int32, device="cuda")
                    pos = torch.arange(c0, c0 + 32768, dtype=torch.int32, device="cuda")
                    gw.gw_kv_append(pool.desc, None, v, si, pos, 32768, pt, stride, cos, sin)
            q = torch.randn(8, 32, 512, device="cuda", generator=g).to(torch.bfloat16)
            dc = RT.DeviceCase(pool, q, None, RT.i32_dev(lens), pt, stride, 8, 8, 1, 131072, 32, 512 ** -0.5, None)
            for _ in range(2):
                RT.attend(dc)
            buf.zero_()
            RT.attend(dc)
            torch.cuda.synchronize()
            rows = buf.view(-1, SLOTS).cpu().numpy().astype(np.uint64)
            raw[f"big_{'e4m3' if fp8 else 'bf16'}"] = rows
            lines.append(summarize(f"global decode 8 x 131072 ({label})", rows, 1, "pairs", 4, 5))
            del pool, dc
            torch.cuda.empty_cache()
    L.gw_trace_buffer(None)
    if dump:
        np.savez(dump, **raw)
    return "\n".join(lines)


if __name__ == "__main__":
    dump = sys.argv[sys.argv.index("--dump") + 1] if "--dump" in sys.argv else None
    if "--prefill" in sys.argv:
        print(run_prefill(dump=dump), flush=True)
    else:
        print(run(big="--big" in sys.argv, dump=dump), flush=True)
