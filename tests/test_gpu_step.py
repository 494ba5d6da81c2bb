"""The 60-layer hybrid step at full size, in the launch configuration that
bench.py times (one HIP graph of every layer's attention call, each call
appending its rows' own tokens first), checked against the CPU oracle on
layers 0 and 58 (local) and 5 and 59 (global), each of which writes its own
output buffer.

Workloads: the decode-only step bench.py reports as its headline (16 decode
slots with seeded contexts in [2048, 8192], one row each, no q_indptr), the
mixed step with 4 new 512-token prompts (pegainfer "Gemma 4" page,
Scheduling: prompt rows share the step with the decode rows), and the same
step with the prompt rows as a 512-token chunk after a cached 3584-token
prefix (chunked prefill against cached context); the decode and the mixed
step also with both families' pools in e4m3 (the oracle then takes the
e4m3 code of every stored element).  The oracle sees only the
seeded draws of the layer (q, the step's new K/V and the prior context K/V,
all bf16) and rotates and rounds them itself; no value comes from the GPU
path.  Every decode row is compared, and a sample of prompt rows (first,
last, and rows on both sides of a page edge).
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import attention as OA
from oracle import codecs as OC
from oracle import rope as OR
from tests.oracle_side import compare

pytestmark = pytest.mark.gpu

# (prompt, row) pairs sampled from the step; every decode row is compared
PROMPT_SAMPLE = [(0, 0), (0, 15), (0, 16), (0, 511), (2, 200), (3, 383)]
# two local and two global layers: the first and the last of each family
CHECK_LAYERS = (0, 5, 58, 59)


def _host(t):
    import torch
    return None if t is None else t.to(torch.float32).cpu().numpy().astype(np.float64)


def _layer_host(st, layer: int):
    """The layer's seeded draws on the host (fp64) and the step's token lists."""
    from paged_hybrid_kv_amd.synth import layer_draws, step_tokens
    sh = st.shape
    local = not sh.is_global(layer)
    d = layer_draws(sh, layer, st.with_prompts, "cuda")
    h = {k: _host(v) for k, v in vars(d).items()}
    return h, step_tokens(sh, st.with_prompts, local)


def _sequence_kv(st, layer: int, s: int, host):
    """Oracle K, V [L][Hkv][D] of sequence s in layer `layer` (NaN where the
    step's pool holds no token) and the oracle q rows of s."""
    sh = st.shape
    local = not sh.is_global(layer)
    h, (new_s, new_p, pri_s, pri_p) = host
    L = int(st.lens[s])
    sel_new, sel_pri = new_s == s, pri_s == s
    pos = np.concatenate([pri_p[sel_pri], new_p[sel_new]])
    v = OC.bf16_round(np.concatenate([h["v_prior"][sel_pri], h["v_new"][sel_new]]))
    if local:
        k = OC.bf16_round(np.concatenate([h["k_prior"][sel_pri], h["k_new"][sel_new]]))
        k = OC.bf16_round(OR.rotate_local(k, pos[:, None]))
        K = np.full((L,) + k.shape[1:], np.nan)
        V = np.full((L,) + v.shape[1:], np.nan)
    else:
        k_rot = OC.bf16_round(OR.rotate_global(v, pos)[:, :128])
        k = OA.k_from_compressed(v, k_rot)[:, None, :]
        v = v[:, None, :]
        K = np.full((L, 1, 512), np.nan)
        V = np.full((L, 1, 512), np.nan)
    from paged_hybrid_kv_amd import gw
    if (st.local_kv_dtype if local else st.global_kv_dtype) == gw.GW_KV_E4M3:
        # an e4m3 pool holds the e4m3 code of every stored bf16 element
        k = OC.e4m3_decode(OC.e4m3_encode(k))
        v = OC.e4m3_decode(OC.e4m3_encode(v))
    K[pos] = k
    V[pos] = v
    indptr = np.concatenate([[0], np.cumsum(st.q_len)])
    q = OC.bf16_round(h["q"][indptr[s]:indptr[s + 1]])
    return K, V, q, int(indptr[s])


def _check_layer(st, layer: int, out):
    sh = st.shape
    local = not sh.is_global(layer)
    window = sh.window if local else None
    D = sh.local_head_dim if local else sh.global_head_dim
    scale = 1.0 / np.sqrt(D)
    gpu = out.cpu().numpy()
    picks = {s: [0] for s in range(sh.decode_slots)}
    if st.with_prompts:
        for i, r in PROMPT_SAMPLE:
            picks.setdefault(sh.decode_slots + i, []).append(r)
    worst = 0.0
    host = _layer_host(st, layer)
    for s, rows in picks.items():
        K, V, q, row0 = _sequence_kv(st, layer, s, host)
        L, ql = int(st.lens[s]), int(st.q_len[s])
        rows = np.array(sorted(set(rows)))
        ref = OA.attend(q[rows], K, V, L - ql + rows, scale, window)
        mx, _, _ = compare(gpu[row0 + rows], ref, f"layer {layer} seq {s} rows {list(rows)}")
        worst = max(worst, mx)
    return worst


def _run_and_check(shape, label, with_prompts=True, e4m3=False):
    import torch
    from paged_hybrid_kv_amd import gw
    from paged_hybrid_kv_amd.step import HybridStep
    dt = gw.GW_KV_E4M3 if e4m3 else gw.GW_KV_BF16
    st = HybridStep(shape=shape, with_prompts=with_prompts, local_kv_dtype=dt, global_kv_dtype=dt)
    st.capture()
    for _ in range(2):
        st.replay()
    torch.cuda.synchronize()
    sh = st.shape
    assert [sh.is_global(l) for l in CHECK_LAYERS] == [False, True, False, True]
    errs = []
    for layer in CHECK_LAYERS:
        print(f"{label}: checking layer {layer}", flush=True)
        errs.append(_check_layer(st, layer, st.layer_out(layer)))
    print(f"{label}: max abs err " + ", ".join(f"layer {l} {e:.2e}" for l, e in zip(CHECK_LAYERS, errs)),
          flush=True)


def test_decode_step_graph_parity():
    # the headline step exactly as bench.py times it: decode rows only
    _run_and_check(None, "decode step", with_prompts=False)


def test_hybrid_step_graph_sampled_parity():
    _run_and_check(None, "mixed step")


def test_hybrid_step_chunked_prefill_sampled_parity():
    # the prompt rows are the last 512-token chunk of 4096-token prompts
    # whose first 3584 tokens are already cached: each row attends a full
    # local window, or 3585..4096 global keys, the cached prefix included
    from paged_hybrid_kv_amd.synth import HybridShape
    _run_and_check(HybridShape(prompt_prefix=3584), "hybrid step, chunk after a 3584-token prefix")


def test_decode_step_e4m3_graph_parity():
    # the headline step with both families' pools in e4m3 (pegainfer PR
    # #1012, Description: the opt-in fp8 pool; here the global family too)
    _run_and_check(None, "decode step, e4m3 pools", with_prompts=False, e4m3=True)


def test_hybrid_step_e4m3_graph_sampled_parity():
    _run_and_check(None, "mixed step, e4m3 pools", e4m3=True)
