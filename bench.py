#!/usr/bin/env python3
"""Benchmark of the paged hybrid-KV decode attention path on one MI355X.

Workload: the 60-layer hybrid decode step of a Gemma 4-style stack -- layer
i global iff (i+1) % 6 == 0 or i == 59 (10 global, 50 local); local layers
hd256, 16 q / 8 KV heads, window 1024, bf16 pool holding the window's
pages; global layers hd512, 32 q / 1 KV head, tied K/V in the compressed
record (V + rotated quarter of K).  16 decode slots with contexts drawn in
[2048, 8192] (seed 5), every layer's data N(0,1) from seed 5000 + layer,
drawn and appended before timing.  A step = for every layer: append the
step's new token per slot (RoPE + store) then paged decode attention of the
16 rows.  The step is captured once as a HIP graph and replayed.

value = algorithmic decode KV bytes of one step (50 local layers x 16 slots x
1024 tokens x 8 KiB + 10 global layers x sum(L) x 1280 B) / step time.
The mixed step (the same plus 4 new 512-token prompts whose causal rows are
computed in the same step) is reported beside it when served.

Prints one JSON line.  --gpus N > 1 is refused: the path runs on one GPU.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
METRIC = "decode-attn KV HBM GB/s (% of peak) + tok/s, 16 slots x 8K hybrid step"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def time_events(fn, iters):
    """Average ms of fn() over iters, with HIP events on torch's current stream."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


COUNTER_FILE = os.path.join(ROOT, "profiles", "local_decode_hbm_counters.json")
LOCAL_KERNEL_SOURCES = ["gw_local.hip", "gw_device.h", "gw_plan.h", "gw_kernels.h"]


def local_kernel_hash():
    """sha256 over the sources the local decode kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for name in LOCAL_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_hybrid_kv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the local decode kernel from the committed
    counter summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or
    None when the kernel's sources changed since the counters were taken."""
    try:
        with open(COUNTER_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_sha256") != local_kernel_hash():
        return None
    return int(c["fetch_bytes_per_launch"] + c["write_bytes_per_launch"])


def dominant_kernel(step, rounds):
    """Local decode attention (50 of 60 layers, most of the KV bytes), called
    as the step calls it (the row's own token appended in the call): average
    duration of one call, timed over all local layers so that consecutive
    calls read different pools (no reuse through the 256 MB last-level cache).
    Re-appending a token writes the same bytes to the same slot."""
    local_layers = [L for L in step.layers if L["local"]]

    def sweep():
        for L in local_layers:
            step.attend(L, append=True)

    sweep()
    ms = time_events(sweep, rounds) / len(local_layers)
    nbytes = step.local_decode_kv_bytes_per_layer()
    achieved = nbytes / (ms * 1e-3)
    return {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM, 4), "traffic": measured_traffic(),
            "kernel": "local_decode_kernel<2,false> (gw_decode_attn_local)",
            "bytes_per_launch": nbytes, "avg_launch_us": round(ms * 1e3, 2)}


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of nbytes, reps times: under a counter
    run it shows what FETCH_SIZE / WRITE_SIZE read for exactly nbytes moved
    each way."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    log(f"copy calibration: {reps} x {nbytes} B device copy")


def cpu_baseline(step):
    """The oracle as it stands, on a bounded sample of the same workload:
    the decode rows of layers 0 and 1 (local) and 5 (global)."""
    import numpy as np
    import torch
    from oracle import attention as OA, codecs as OC, rope as OR
    from paged_hybrid_kv_amd.synth import layer_draws, step_tokens

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    sh = step.shape
    layers = [0, 1, 5]
    host = {}
    for l in layers:
        d = layer_draws(sh, l, False, "cuda")
        host[l] = {k: (None if v is None else v.float().cpu().numpy())
                   for k, v in vars(d).items()}
    torch.cuda.synchronize()
    nbytes = 0
    t0 = time.perf_counter()
    for l in layers:
        local = not sh.is_global(l)
        ns, npos, ps, pp = step_tokens(sh, False, local)
        h = host[l]
        for s in range(sh.decode_slots):
            L = int(sh.decode_lens[s])
            sel_p, sel_n = ps == s, ns == s
            pos = np.concatenate([pp[sel_p], npos[sel_n]])
            v = OC.bf16_round(np.concatenate([h["v_prior"][sel_p], h["v_new"][sel_n]]).astype(np.float64))
            q = OC.bf16_round(h["q"][s:s + 1].astype(np.float64))
            if local:
                k = OC.bf16_round(np.concatenate([h["k_prior"][sel_p], h["k_new"][sel_n]]).astype(np.float64))
                k = OC.bf16_round(OR.rotate_local(k, pos[:, None]))
                lo = int(pos[0])
                K = np.full((L, sh.local_kv_heads, 256), np.nan)
                V = np.full((L, sh.local_kv_heads, 256), np.nan)
                K[pos], V[pos] = k, v
                OA.attend_sequence(q, K, V, 1 / 16, sh.window)
                nbytes += min(L, sh.window) * sh.local_kv_heads * 256 * 4
                del lo
            else:
                k_rot = OC.bf16_round(OR.rotate_global(v, pos)[:, :128])
                K = OA.k_from_compressed(v, k_rot)[:, None, :]
                OA.attend_sequence(q, K, v[:, None, :], 512 ** -0.5, None)
                nbytes += L * 1280
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": "decode rows (16 slots) of layers 0, 1 (local) and 5 (global) of the same step: "
                      "fp64 rotation, bf16 rounding and naive masked softmax over contiguous K/V; "
                      f"{nbytes} algorithmic KV bytes; os.cpu_count()={os.cpu_count()}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-graph", action="store_true", help="replay the step eagerly")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-rounds", type=int, default=10)
    ap.add_argument("--no-mixed", action="store_true", help="skip the step with prompt rows")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy three times (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU path only (no sharding, no collectives); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_hybrid_kv_amd import gw
    from paged_hybrid_kv_amd.runtime import require_gpu
    from paged_hybrid_kv_amd.step import HybridStep

    require_gpu()
    log(f"{gw.gw_version()} on {torch.cuda.get_device_name(0)}")
    t0 = time.time()
    step = HybridStep(with_prompts=False)
    torch.cuda.synchronize()
    log(f"decode step built in {time.time() - t0:.1f}s (context appended)")
    if not args.no_graph:
        step.capture()
    for _ in range(args.warmup):
        step.replay()
    torch.cuda.synchronize()
    ms = time_events(step.replay, args.steps)
    dec_bytes = step.decode_kv_bytes()
    value = dec_bytes / (ms * 1e-3) / 1e9
    log(f"decode step: {ms:.3f} ms, {value:.0f} GB/s decode KV ({value * 1e9 / PEAK_HBM * 100:.1f}% of peak)")

    roof = dominant_kernel(step, args.kernel_rounds)
    log(f"dominant kernel: {roof['avg_launch_us']} us/launch, {roof['achieved']} GB/s ({roof['frac'] * 100:.1f}%)")

    mixed = None
    try:
        if args.no_mixed:
            raise gw.GwError(0, "skipped (--no-mixed)")
        ms_step = HybridStep(with_prompts=True)
        if not args.no_graph:
            ms_step.capture()
        for _ in range(args.warmup):
            ms_step.replay()
        mms = time_events(ms_step.replay, args.steps)
        mb = ms_step.mixed_step_bytes()
        mixed = {"ms_per_step": round(mms, 4), "decode_tok_s": round(16 / (mms * 1e-3), 1),
                 "rows_per_s": round(ms_step.rows / (mms * 1e-3), 1), "rows": ms_step.rows,
                 "algorithmic_bytes": mb,
                 "GB_per_s": round(mb["total"] / (mms * 1e-3) / 1e9, 1),
                 "pct_of_peak": round(mb["total"] / (mms * 1e-3) / PEAK_HBM * 100, 2)}
        del ms_step
    except gw.GwError as e:
        mixed = {"served": False, "reason": e.message}
    torch.cuda.empty_cache()

    if args.copy_calib:
        copy_calibration()

    cpu = None if args.no_cpu_baseline else cpu_baseline(step)
    if cpu:
        log(f"cpu baseline: {cpu['value']} GB/s over {cpu['seconds']} s on {cpu['cores']} threads")

    sh = step.shape
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "pct_of_peak": round(value * 1e9 / PEAK_HBM * 100, 2),
        "decode_tok_s": round(sh.decode_slots / (ms * 1e-3), 1),
        "decode_kv_bytes_per_step": dec_bytes,
        "config": {"workload": "gemma4 hybrid decode step: 60 layers (50 local hd256 16q/8kv window 1024 "
                               "bf16 pool, 10 global hd512 32q/1kv tied compressed pool), 16 slots, "
                               "contexts U[2048,8192] seed 5, 16-token pages",
                   "layers": sh.num_layers, "slots": sh.decode_slots,
                   "contexts": [int(x) for x in sh.decode_lens], "graph": not args.no_graph},
        "roofline": roof,
        "mixed_step": mixed,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
