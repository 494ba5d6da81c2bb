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
computed in the same step) is reported beside it, and so is the same step
with the prompt rows as a 512-token chunk after a cached 3584-token prefix
(chunked prefill: every row attends a full local window and 3585..4096
global keys), and the decode step with e4m3 pools: the local family's only
(the opt-in fp8 pool of pegainfer PR #1012) and both families'.

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
LOCAL_KERNEL_SOURCES = ["gw_local.hip", "gw_device.h", "gw_plan.h", "gw_kernels.h", "gw_rows_append.h"]


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
    """The oracle as it stands, on a bounded sample of the same workload
    (about 10-15 s of host work): the decode rows of layers 0-4 and 6
    (local) and 5 and 11 (global)."""
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
    layers = [0, 1, 2, 3, 4, 5, 6, 11]
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
                K = np.full((L, sh.local_kv_heads, 256), np.nan)
                V = np.full((L, sh.local_kv_heads, 256), np.nan)
                K[pos], V[pos] = k, v
                OA.attend_sequence(q, K, V, 1 / 16, sh.window)
                nbytes += min(L, sh.window) * sh.local_kv_heads * 256 * 4
            else:
                k_rot = OC.bf16_round(OR.rotate_global(v, pos)[:, :128])
                K = OA.k_from_compressed(v, k_rot)[:, None, :]
                OA.attend_sequence(q, K, v[:, None, :], 512 ** -0.5, None)
                nbytes += L * 1280
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"decode rows (16 slots) of layers {', '.join(str(l) for l in layers if not sh.is_global(l))} "
                      f"(local) and {', '.join(str(l) for l in layers if sh.is_global(l))} (global) of the same step: "
                      "fp64 rotation, bf16 rounding and naive masked softmax over contiguous K/V; "
                      f"{nbytes} algorithmic KV bytes; os.cpu_count()={os.cpu_count()}"}


def config_throughput(iters=30, oracle=True):
    """Decode-attention throughput of the three single-family workloads at
    their full sizes (the parity tests' cases; the page tables come from the
    same seeded recipes, the pools are filled on the device with torch's
    seeded generator): local bf16 (16 slots, contexts U[1024, 8192], window
    1024, 16 q / 8 KV heads), global tied (8 slots x 131072 tokens, 32 q / 1
    KV head, compressed and full records, in bf16 and in e4m3 pools) and
    local e4m3 (64 slots x 8192); and the page copy of the prefix cache
    (4096 local bf16 pages, read and written once).
    Calls run back to back over pool replicas whose total exceeds the 256 MB
    last-level cache; returns {name: {us, GB_s, pct_of_peak, tok_s, bytes}}."""
    import numpy as np
    import torch
    from paged_hybrid_kv_amd import gw, runtime as RT, synth as SY

    dev = "cuda"

    def local_pool(lens, fp8, seed, rep):
        rng = np.random.default_rng(seed)
        lens = lens(rng) if callable(lens) else np.asarray(lens)
        seqs = SY.make_page_table(rng, lens)
        dt = gw.GW_KV_E4M3 if fp8 else gw.GW_KV_BF16
        pool = RT.Pool(gw.GW_FAMILY_LOCAL, dt, seqs.num_pages, 8, 256, dev)
        pt, stride = RT.i32_dev(seqs.page_table), seqs.page_table.shape[1]
        max_len = int(lens.max())
        cos, sin = RT.rope_tables(max_len, 256, 256, RT.LOCAL_THETA)
        g = torch.Generator(device=dev)
        g.manual_seed(1000 * seed + rep)
        for s, L in enumerate(lens):           # the window's tokens (and the rest of its first page)
            lo = max(0, int(L) - 1024) // 16 * 16
            n = int(L) - lo
            k = (torch.randn(n, 8, 256, device=dev, generator=g) * 0.5).to(torch.bfloat16)
            v = (torch.randn(n, 8, 256, device=dev, generator=g) * 0.5).to(torch.bfloat16)
            si = torch.full((n,), s, dtype=torch.int32, device=dev)
            pos = torch.arange(lo, int(L), dtype=torch.int32, device=dev)
            gw.gw_kv_append(pool.desc, k, v, si, pos, n, pt, stride, cos, sin)
        q = (torch.randn(len(lens), 16, 256, device=dev, generator=g) * 0.5).to(torch.bfloat16)
        return RT.DeviceCase(pool, q, None, RT.i32_dev(lens), pt, stride, len(lens), len(lens), 1, max_len,
                             16, 1 / 16, 1024)

    def global_pool(compressed, fp8=False):
        rng = np.random.default_rng(3)
        lens = np.full(8, 131072)
        seqs = SY.make_page_table(rng, lens)
        fam = gw.GW_FAMILY_GLOBAL_COMPRESSED if compressed else gw.GW_FAMILY_GLOBAL_FULL
        pool = RT.Pool(fam, gw.GW_KV_E4M3 if fp8 else gw.GW_KV_BF16, seqs.num_pages, 1, 128, dev)
        pt, stride = RT.i32_dev(seqs.page_table), seqs.page_table.shape[1]
        cos, sin = RT.rope_tables(131072, 128, 512, RT.GLOBAL_THETA)
        g = torch.Generator(device=dev)
        g.manual_seed(3000)
        for s in range(8):
            for c0 in range(0, 131072, 32768):
                v = torch.randn(32768, 512, device=dev, generator=g).to(torch.bfloat16)
                si = torch.full((32768,), s, dtype=torch.int32, device=dev)
                pos = torch.arange(c0, c0 + 32768, dtype=torch.int32, device=dev)
                gw.gw_kv_append(pool.desc, None, v, si, pos, 32768, pt, stride, cos, sin)
        q = torch.randn(8, 32, 512, device=dev, generator=g).to(torch.bfloat16)
        return RT.DeviceCase(pool, q, None, RT.i32_dev(lens), pt, stride, 8, 8, 1, 131072, 32, 512 ** -0.5, None)

    def timed(dcs, nbytes, slots, keep=None):
        ws = RT.Workspace()
        outs = [RT.attend(dc, ws=ws) for dc in dcs]
        torch.cuda.synchronize()
        if keep is not None:
            keep.append(outs[0].clone())
        ms = time_events(lambda: [RT.attend(dc, out=o, ws=ws) for dc, o in zip(dcs, outs)], iters) / len(dcs)
        return {"us": round(ms * 1e3, 2), "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "pct_of_peak": round(nbytes / (ms * 1e-3) / PEAK_HBM * 100, 2),
                "tok_s": round(slots / (ms * 1e-3), 1), "bytes": nbytes}

    res = {}
    c2_lens = lambda r: r.integers(1024, 8192, size=16, endpoint=True)
    lens2 = c2_lens(np.random.default_rng(2))
    c2 = [local_pool(c2_lens, False, 2, r) for r in range(4)]
    res["local_bf16"] = timed(c2, int(sum(min(int(L), 1024) for L in lens2)) * 8 * 256 * 2 * 2, 16)
    del c2
    torch.cuda.empty_cache()
    for fp8 in (False, True):
        kept = []
        for compressed in (True, False):
            dc = global_pool(compressed, fp8)
            res["global_" + ("compressed" if compressed else "full") + ("_e4m3" if fp8 else "")] = timed(
                [dc], 8 * 131072 * (640 if compressed else 1024) * (1 if fp8 else 2), 8, kept)
            del dc
            torch.cuda.empty_cache()
        # the two records of the same draws give bit-identical outputs
        res["global_compressed" + ("_e4m3" if fp8 else "")]["compressed_equals_full"] = bool(torch.equal(kept[0], kept[1]))
        del kept
    # prefix-cache page copies: 4096 local bf16 pages (512 MiB) from a cache
    # pool into a live pool, in a shuffled order; bytes counted once each way
    src = RT.Pool(gw.GW_FAMILY_LOCAL, gw.GW_KV_BF16, 4096, 8, 256, dev, fill_byte=1)
    dst = RT.Pool(gw.GW_FAMILY_LOCAL, gw.GW_KV_BF16, 4096, 8, 256, dev, fill_byte=0)
    perm = np.random.default_rng(6).permutation(4096).astype(np.int32)
    ids_s, ids_d = RT.i32_dev(np.arange(4096, dtype=np.int32)), RT.i32_dev(perm)
    gw.gw_copy_pages(dst.desc, src.desc, ids_d, ids_s, 4096)
    ms = time_events(lambda: gw.gw_copy_pages(dst.desc, src.desc, ids_d, ids_s, 4096), iters)
    nbytes = 2 * 4096 * src.page_bytes
    res["copy_pages"] = {"us": round(ms * 1e3, 2), "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                         "pct_of_peak": round(nbytes / (ms * 1e-3) / PEAK_HBM * 100, 2),
                         "tok_s": round(4096 * 16 / (ms * 1e-3), 1), "bytes": nbytes}
    del src, dst
    torch.cuda.empty_cache()
    c4 = [local_pool([8192] * 64, True, 4, r) for r in range(2)]
    res["local_fp8"] = timed(c4, 64 * 1024 * 8 * 256 * 2, 64)
    del c4
    torch.cuda.empty_cache()
    if oracle:
        for k, o in config_oracle().items():
            res[k]["cpu_baseline"] = o
    for k, v in res.items():
        log(f"{k}: {v['us']} us/call, {v['GB_s']} GB/s ({v['pct_of_peak']}% of peak), {v['tok_s']} tok/s"
            + (f"; oracle {v['cpu_baseline']['value']} GB/s" if "cpu_baseline" in v else ""))
    return res


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def config_oracle():
    """The oracle as it stands on a bounded sample of each single-family
    workload (same shapes, value distributions and rotation as the timed
    calls; the sample's K/V come from the seeded recipes of the parity
    tests): the local bf16 workload's first 4 slots, one 131072-token slot of
    the global tied workload (compressed record, K rebuilt from V and the
    rotated quarter), and 4 of the 64 local e4m3 slots.  Returns
    {name: cpu_baseline}, GB/s of the same algorithmic bytes."""
    import numpy as np
    from oracle import attention as OA, codecs as OC, rope as OR
    from paged_hybrid_kv_amd import synth as SY

    def timed_oracle(case, seqs, per_seq_bytes, label):
        # timed: the oracle's own rounding, rotation, e4m3 decode and attention
        t0 = time.perf_counter()
        nbytes = 0
        for s in seqs:
            L = int(case.seqs.lens[s])
            sel = case.tok_seq == s
            pos = case.tok_pos[sel]
            q = OC.bf16_round(case.q[s:s + 1].astype(np.float64))
            if hasattr(case, "window"):
                k = OC.bf16_round(case.k[sel].astype(np.float64))
                v = OC.bf16_round(case.v[sel].astype(np.float64))
                k = OC.bf16_round(OR.rotate_local(k, pos[:, None]))
                if case.fp8:
                    k = OC.e4m3_decode(OC.e4m3_encode(k))
                    v = OC.e4m3_decode(OC.e4m3_encode(v))
                K = np.full((L,) + k.shape[1:], np.nan)
                V = np.full((L,) + v.shape[1:], np.nan)
                K[pos], V[pos] = k, v
                OA.attend_sequence(q, K, V, case.scale, case.window)
            else:
                v = OC.bf16_round(case.v[sel].astype(np.float64))
                k_rot = OC.bf16_round(OR.rotate_global(v, pos)[:, :128])
                K = OA.k_from_compressed(v, k_rot)[:, None, :]
                OA.attend_sequence(q, K, v[:, None, :], case.scale, None)
            nbytes += per_seq_bytes(L)
        dt = time.perf_counter() - t0
        return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": _threads(), "kind": "oracle",
                "seconds": round(dt, 2), "sample": f"{label}; {nbytes} algorithmic KV bytes; "
                                                   f"os.cpu_count()={os.cpu_count()}"}

    out = {}
    lens2 = np.random.default_rng(2).integers(1024, 8192, size=16, endpoint=True)[:4]
    c2 = SY.local_case("oracle sample", 2, lens2, window=1024, num_q_heads=16, num_kv_heads=8, q_scale=0.5,
                       kv_scale=0.5, rope=True, fill_window_only=True)
    out["local_bf16"] = timed_oracle(c2, range(4), lambda L: min(L, 1024) * 8 * 256 * 2 * 2,
                                     "4 of the 16 local bf16 slots (window 1024, 16 q / 8 KV heads), fp64 rotation "
                                     "and naive masked softmax")
    c3 = SY.global_case("oracle sample", 3, [131072], num_q_heads=32, rope=True)
    out["global_compressed"] = timed_oracle(c3, range(1), lambda L: L * 1280,
                                            "1 of the 8 global slots (131072 tokens, 32 q heads, K rebuilt from "
                                            "V and the rotated quarter)")
    c4 = SY.local_case("oracle sample", 4, [8192] * 4, window=1024, num_q_heads=16, num_kv_heads=8, q_scale=0.5,
                       kv_scale=0.5, rope=True, fp8=True, fill_window_only=True)
    out["local_fp8"] = timed_oracle(c4, range(4), lambda L: min(L, 1024) * 8 * 256 * 2,
                                    "4 of the 64 local e4m3 slots (8192 tokens, window 1024), e4m3 decode of the "
                                    "stored codes")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-graph", action="store_true", help="replay the step eagerly")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-rounds", type=int, default=10)
    ap.add_argument("--no-mixed", action="store_true", help="skip the step with prompt rows")
    ap.add_argument("--no-e4m3-steps", action="store_true", help="skip the decode step with e4m3 pools")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the local bf16, global tied and local e4m3 workloads at full size")
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

    def prompt_step(shape, label):
        ms_step = HybridStep(shape=shape, with_prompts=True)
        if not args.no_graph:
            ms_step.capture()
        for _ in range(args.warmup):
            ms_step.replay()
        mms = time_events(ms_step.replay, args.steps)
        mb = ms_step.mixed_step_bytes()
        fl = ms_step.prompt_flops()
        res = {"ms_per_step": round(mms, 4), "decode_tok_s": round(16 / (mms * 1e-3), 1),
               "rows_per_s": round(ms_step.rows / (mms * 1e-3), 1), "rows": ms_step.rows,
               "prompt_prefix": ms_step.shape.prompt_prefix,
               "algorithmic_bytes": mb,
               "GB_per_s": round(mb["total"] / (mms * 1e-3) / 1e9, 1),
               "pct_of_peak": round(mb["total"] / (mms * 1e-3) / PEAK_HBM * 100, 2),
               "prompt_row_gflop": round(fl / 1e9, 1)}
        log(f"{label}: {mms:.3f} ms, {res['GB_per_s']} GB/s ({res['pct_of_peak']}% of peak), "
            f"{res['prompt_row_gflop']} GFLOP of prompt-row products")
        del ms_step
        torch.cuda.empty_cache()
        return res

    mixed = chunked = None
    if args.no_mixed:
        mixed = chunked = {"served": False, "reason": "skipped (--no-mixed)"}
    else:
        from paged_hybrid_kv_amd.synth import HybridShape
        for key, shape, label in (("mixed", None, "mixed step"),
                                  ("chunked", HybridShape(prompt_prefix=3584),
                                   "mixed step, prompt chunk after a 3584-token cached prefix")):
            try:
                r = prompt_step(shape, label)
            except gw.GwError as e:
                r = {"served": False, "reason": e.message}
            if key == "mixed":
                mixed = r
            else:
                chunked = r

    def e4m3_decode_step(local_dt, global_dt, label):
        """The headline step with e4m3 pools (pegainfer PR #1012, Verification:
        the opt-in fp8 local pool measured against bf16 at the same
        concurrency): its time, tok/s and the bytes its pools hold."""
        st2 = HybridStep(with_prompts=False, local_kv_dtype=local_dt, global_kv_dtype=global_dt)
        if not args.no_graph:
            st2.capture()
        for _ in range(args.warmup):
            st2.replay()
        ems = time_events(st2.replay, args.steps)
        kvb = st2.decode_kv_bytes()
        res = {"ms_per_step": round(ems, 4), "decode_tok_s": round(st2.shape.decode_slots / (ems * 1e-3), 1),
               "decode_kv_bytes_per_step": kvb, "GB_per_s": round(kvb / (ems * 1e-3) / 1e9, 1),
               "pct_of_peak": round(kvb / (ems * 1e-3) / PEAK_HBM * 100, 2),
               "speedup_vs_bf16_step": round(ms / ems, 3)}
        log(f"{label}: {ems:.3f} ms, {res['decode_tok_s']} tok/s ({res['speedup_vs_bf16_step']}x the bf16 step), "
            f"{res['GB_per_s']} GB/s of e4m3 KV")
        del st2
        torch.cuda.empty_cache()
        return res

    e4m3_steps = None
    if not args.no_e4m3_steps:
        e4m3_steps = {
            "local_e4m3": e4m3_decode_step(gw.GW_KV_E4M3, gw.GW_KV_BF16, "decode step, local pools e4m3"),
            "local_and_global_e4m3": e4m3_decode_step(gw.GW_KV_E4M3, gw.GW_KV_E4M3,
                                                      "decode step, both families' pools e4m3"),
        }

    if args.copy_calib:
        copy_calibration()

    configs = None if args.no_configs else config_throughput(oracle=not args.no_cpu_baseline)

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
                               "bf16 pool, 10 global hd512 32q/1kv tied compressed pool), 16 decode slots, "
                               "contexts U[2048,8192] seed 5, 16-token pages; decode rows only (0 prompt rows: "
                               "the same step with 4 x 512 prompt rows is mixed_step)",
                   "prompt_rows": 0,
                   "layers": sh.num_layers, "slots": sh.decode_slots,
                   "contexts": [int(x) for x in sh.decode_lens], "graph": not args.no_graph},
        "roofline": roof,
        "mixed_step": mixed,
        "chunked_prefill_step": chunked,
        "decode_step_e4m3": e4m3_steps,
        "cpu_baseline": cpu,
    }
    if configs is not None:
        line["other_configs"] = configs
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
