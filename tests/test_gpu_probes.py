"""Bit-exact index probes over multi-split ranges, both families.

A dominant key: K[j*] is set along one q head's direction, 200 / |q| times
q, so that head's score for j* exceeds every other score by more than 120
(checked on the host for each probe); every other weight then underflows to
exactly 0 in fp32 (2^-173 < 2^-149), the weight of j* is exactly 1, and the
head's output must equal V[j*] bit for bit -- whichever split, wave, page or
merge step handles j*.  Each q head of a sequence carries its own probe (the
local family: at a distinct position of its KV head; the global family: all
32 heads on the one KV head), so a sequence checks up to 32 positions.

Positions probed (pegainfer "Gemma 4" page, Scheduling: a 1024-token window;
pegainfer PR #1012, Verification: the window-edge waypoint):
  local  -- both window ends, one token of every virtual page (its first,
            last or middle slot, in turn), both sides of every split
            boundary, and every slot of the merged partial page at the two
            ends of a window that does not start on a page boundary;
  global -- the first and last token, both sides of every split boundary
            (7 to 63 splits per row), and one token of every page for the
            shorter rows.
Lengths cover aligned windows, windows that wrap (merged end pages), rows
shorter than the window, and global rows of 2000 to 20000 tokens.  Every
case runs with the pool already holding the rows' tokens and with each row's
own token appended inside the attention call.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_hybrid_kv_amd import runtime as RT, synth as SY

from .oracle_side import global_seq, local_seq

pytestmark = pytest.mark.gpu

MARGIN = 120.0    # least gap between the probe's score and any other (natural log units, scaled)


# ------------------------------------------------------------------ plans --
# The probe positions come from the plan's own definition of splits (a
# balanced cut of the range's pages: part i starts at floor(n i / k)), so
# that every boundary is probed on both sides.
def _cut(n, k):
    return [n * i // k for i in range(k + 1)]


def _local_nsplit(nv, group):
    per = 17 if group >= 4 else 33
    return max(1, min(16, -(-nv // per)))


def _global_nsplit(n):
    k = max(1, min(64, -(-n // 20)))
    return max(k, -(-n // 256))


def local_positions(L, window, group):
    """Probe positions for a decode row at p = L - 1 (see module doc)."""
    p = L - 1
    lo = max(0, p - window + 1)
    pg0, pgl = lo // 16, p // 16
    wrap = pgl > pg0 and p % 16 < lo % 16
    # virtual pages: v = 0 is the merged pair (wrap) or page pg0; v >= 1 is pg0 + v
    nv = pgl - pg0 if wrap else pgl - pg0 + 1

    def tokens(v):
        if v == 0 and wrap:
            return list(range(lo, 16 * pg0 + 16)) + list(range(16 * pgl, p + 1))
        pg = pg0 + v
        return [t for t in range(16 * pg, 16 * pg + 16) if lo <= t <= p]

    pos = {lo, min(lo + 1, p), max(p - 1, lo), p}
    for v in range(nv):
        t = tokens(v)
        pos.add(t[[0, -1, len(t) // 2][v % 3]])
    cut = _cut(nv, _local_nsplit(nv, group))
    for b in cut[1:-1]:
        pos.add(tokens(b - 1)[-1])
        pos.add(tokens(b)[0])
    if wrap:
        pos.update(tokens(0))
    return sorted(pos)


def global_positions(L, every_page):
    n = -(-L // 16)
    pos = {0, L - 1}
    cut = _cut(n, _global_nsplit(n))
    for b in cut[1:-1]:
        pos.update({16 * b - 1, 16 * b})
    if every_page:
        for pg in range(n):
            pos.add(min(16 * pg + (0, 15, 7)[pg % 3], L - 1))
    return sorted(pos)


# ------------------------------------------------------------------ local --
LOCAL_LENS = [2048, 2000, 2001, 2008, 2015, 5000, 8192, 1024, 1025, 700, 33]


def local_probe_case(group, fp8, seed):
    """Sequences of the listed lengths, each carrying Hkv x G probes; returns
    (case, probes) with probes[s] = {q head: position}."""
    hkv = 8
    hq = hkv * group
    lens, probes = [], []
    for L in LOCAL_LENS:
        ps = local_positions(L, 1024, group)
        for c0 in range(0, len(ps), hq):
            chunk = ps[c0:c0 + hq]
            lens.append(L)
            # head h gets chunk[h]; the G heads of a KV head get distinct positions
            probes.append({h: chunk[h] for h in range(len(chunk))})
    case = SY.local_case("probes", seed, lens, window=1024, num_q_heads=hq, num_kv_heads=hkv, q_scale=1.0,
                         kv_scale=0.5, rope=False, fp8=fp8, fill_window_only=True)
    for s, pr in enumerate(probes):
        for h, j in pr.items():
            g = h // group
            qd = case.q[s, h].astype(np.float64)
            idx = np.nonzero((case.tok_seq == s) & (case.tok_pos == j))[0][0]
            case.k[idx, g] = (200.0 * qd / np.linalg.norm(qd)).astype(np.float32)
    return case, probes


def _check_local_margins(case, probes, group, kv):
    for s, pr in enumerate(probes):
        K, _ = kv[s]
        q = case.q[s].astype(np.float64)
        L = int(case.seqs.lens[s])
        lo = max(0, L - 1024)
        for h, j in pr.items():
            z = K[lo:L, h // group] @ q[h] * case.scale
            zj = z[j - lo]
            z[j - lo] = -np.inf
            assert zj - np.nanmax(z) > MARGIN, (s, h, j)


def _drop_last_tokens(case):
    """The case without each sequence's last token, and that token's raw K/V."""
    import copy
    last = np.array([np.nonzero((case.tok_seq == s) & (case.tok_pos == int(L) - 1))[0][0]
                     for s, L in enumerate(case.seqs.lens)])
    keep = np.ones(case.tok_seq.shape[0], bool)
    keep[last] = False
    c2 = copy.copy(case)
    c2.tok_seq, c2.tok_pos = case.tok_seq[keep], case.tok_pos[keep]
    if hasattr(case, "k"):
        c2.k = case.k[keep]
    c2.v = case.v[keep]
    return c2, last


@pytest.mark.parametrize("group", [2, 4])
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("in_call", [False, True])
def test_local_multisplit_probes(group, fp8, in_call):
    case, probes = local_probe_case(group, fp8, 300 + group + 10 * fp8)
    kv = [local_seq(case, s) for s in range(len(probes))]   # oracle K, V (fp64) of every sequence
    _check_local_margins(case, probes, group, kv)
    print(f"local probes G={group} fp8={fp8} in_call={in_call}: {len(probes)} sequences, "
          f"{sum(len(p) for p in probes)} probes", flush=True)
    if in_call:
        c2, last = _drop_last_tokens(case)
        dc = RT.upload_local(c2)
        out = RT.attend(dc, k_new=RT.to_bf16_dev(case.k[last]), v_new=RT.to_bf16_dev(case.v[last]))
    else:
        dc = RT.upload_local(case)
        out = RT.attend(dc)
    out = out.cpu().numpy()
    bad = []
    for s, pr in enumerate(probes):
        _, V = kv[s]
        for h, j in pr.items():
            want = V[j, h // group].astype(np.float32)
            if not np.array_equal(out[s, h], want):
                bad.append((int(case.seqs.lens[s]), h, j))
    assert not bad, f"{len(bad)} probes differ from V[j*] (L, head, j*): {bad[:10]}"


# ----------------------------------------------------------------- global --
GLOBAL_LENS = [(2000, True), (2007, True), (4099, True), (8192, False), (20000, False)]


def global_probe_case(fp8, seed):
    lens, probes = [], []
    for L, every in GLOBAL_LENS:
        ps = global_positions(L, every)
        for c0 in range(0, len(ps), 32):
            chunk = ps[c0:c0 + 32]
            lens.append(L)
            probes.append({h: chunk[h] for h in range(len(chunk))})
    case = SY.global_case("probes", seed, lens, num_q_heads=32, rope=False, fp8=fp8)
    for s, pr in enumerate(probes):
        for h, j in pr.items():
            qd = case.q[s, h].astype(np.float64)
            idx = np.nonzero((case.tok_seq == s) & (case.tok_pos == j))[0][0]
            case.v[idx] = (200.0 * qd / np.linalg.norm(qd)).astype(np.float32)   # K = V (tied)
    return case, probes


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("in_call", [False, True])
def test_global_multisplit_probes(fp8, in_call):
    case, probes = global_probe_case(fp8, 400 + 10 * fp8)
    kv = [global_seq(case, s) for s in range(len(probes))]   # oracle K, V (fp64) of every sequence
    for s, pr in enumerate(probes):
        K, _ = kv[s]
        q = case.q[s].astype(np.float64)
        for h, j in pr.items():
            z = K[:, 0] @ q[h] * case.scale
            zj = z[j]
            z[j] = -np.inf
            assert zj - z.max() > MARGIN, (s, h, j)
    print(f"global probes fp8={fp8} in_call={in_call}: {len(probes)} sequences, "
          f"{sum(len(p) for p in probes)} probes", flush=True)
    outs = []
    for compressed in (True, False):
        if in_call:
            c2, last = _drop_last_tokens(case)
            dc = RT.upload_global(c2, compressed=compressed)
            max_len = int(case.seqs.lens.max())
            rope = RT.identity_rope_tables(max_len, 128)
            out = RT.attend(dc, v_new=RT.to_bf16_dev(case.v[last]), rope=rope)
        else:
            dc = RT.upload_global(case, compressed=compressed)
            out = RT.attend(dc)
        outs.append(out.cpu().numpy())
        del dc
        torch.cuda.empty_cache()
    assert np.array_equal(outs[0], outs[1]), "compressed and full records differ"
    bad = []
    for s, pr in enumerate(probes):
        _, V = kv[s]
        for h, j in pr.items():
            if not np.array_equal(outs[0][s, h], V[j, 0].astype(np.float32)):
                bad.append((int(case.seqs.lens[s]), h, j))
    assert not bad, f"{len(bad)} probes differ from V[j*] (L, head, j*): {bad[:10]}"
