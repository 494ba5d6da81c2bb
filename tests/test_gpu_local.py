"""Local family on the GPU: append + paged sliding-window decode attention
(bf16 and e4m3 pools) against the CPU oracle, and the bit-exact gates.

Workloads (paged_hybrid_kv_amd.synth): the tiny 64-token case, the 16-slot
bf16 case with lengths in [1024, 8192], the 64-slot x 8192 e4m3 case, plus
edge cases.  Tolerances: max abs 1e-2, mean abs 1e-3 against the fp64
oracle fed the same bf16 / e4m3-decoded values.
"""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import codecs as OC
from oracle import pool as OP
from paged_hybrid_kv_amd import gw, runtime as RT, synth as SY

from .oracle_side import compare, local_seq, oracle_out, q_rows

pytestmark = pytest.mark.gpu


def run(case, **kw):
    dc = RT.upload_local(case, **kw)
    out = RT.attend(dc)
    torch.cuda.synchronize()
    return dc, out.cpu().numpy()


def rows_of(out, case, s):
    qi = case.q_indptr
    return out[qi[s]:qi[s + 1]]


def check_all(case, out, label):
    ref = oracle_out(case)
    worst = 0.0
    for s, r in ref.items():
        mx, _, _ = compare(rows_of(out, case, s), r, f"{label} seq {s}")
        worst = max(worst, mx)
    return worst


# ------------------------------------------------------------------ parity --
def test_tiny_local():
    case = SY.tiny_local()
    _, out = run(case)
    mx = check_all(case, out, "tiny")
    print(f"tiny_local max abs err {mx:.2e}", flush=True)


@pytest.mark.parametrize("G,Hkv", [(1, 2), (2, 3), (4, 2)])
def test_group_sizes(G, Hkv):
    case = SY.local_case("groups", 10 + G, [37, 300, 1500, 16, 1], window=256, num_q_heads=G * Hkv,
                         num_kv_heads=Hkv, rope=False)
    _, out = run(case)
    check_all(case, out, f"G={G}")


@pytest.mark.parametrize("fp8", [False, True])
def test_edge_lengths(fp8):
    # lengths around page and window edges, windows of 1, short and longer than L
    lens = [1, 2, 15, 16, 17, 31, 32, 33, 255, 256, 257, 1023, 1024, 1025, 1039, 1040, 1041, 3000]
    for W in (1, 7, 16, 100, 1024, 5000):
        case = SY.local_case(f"edges W={W}", 20 + W, lens, window=W, num_q_heads=4, num_kv_heads=2,
                             rope=False, fp8=fp8, kv_scale=0.5, q_scale=0.5)
        _, out = run(case)
        check_all(case, out, f"edges W={W} fp8={fp8}")


def test_local_bf16_exact_inputs():
    # the 16-slot workload's shapes, K stored as drawn (no rotation): the
    # oracle sees exactly the GPU's bf16 values
    case = SY.local_bf16()
    case.rope = False
    _, out = run(case)
    mx = check_all(case, out, "local_bf16/unrotated")
    print(f"local_bf16 (unrotated) max abs err {mx:.2e}", flush=True)


def test_local_bf16_rotated():
    # the full path: K rotated on the GPU in fp32, by the oracle in fp64
    case = SY.local_bf16()
    _, out = run(case)
    mx = check_all(case, out, "local_bf16")
    print(f"local_bf16 max abs err {mx:.2e}", flush=True)


def test_local_fp8_full_size():
    # 64 slots x 8192 tokens, K rotated (theta 1e4) before the e4m3 store, as
    # the 16-slot bf16 workload rotates it: the GPU rotates in fp32, the
    # oracle in fp64, each rounding to bf16 and then to e4m3
    case = SY.local_fp8()
    assert case.rope
    _, out = run(case)
    sample = list(range(0, 64, 7))
    ref = oracle_out(case, sample)
    worst = 0.0
    for s in sample:
        mx, _, _ = compare(rows_of(out, case, s), ref[s], f"local_fp8 seq {s}")
        worst = max(worst, mx)
    print(f"local_fp8 rotated (sampled {len(sample)} slots) max abs err {worst:.2e}", flush=True)


def test_local_fp8_rotated_small():
    case = SY.local_case("fp8 rotated", 41, [2000, 1100, 5000, 64], window=1024, num_q_heads=16,
                         num_kv_heads=8, q_scale=0.5, kv_scale=0.5, rope=True, fp8=True)
    _, out = run(case)
    check_all(case, out, "fp8 rotated")


# --------------------------------------------------------- bit-exact gates --
def dominant_case(fp8, W=64, L=200):
    """One sequence per probe position j*: K[j*] = 200 q/|q| so every other
    weight underflows to 0 and the output must be V[j*] exactly."""
    lo = L - W
    probes = list(range(lo, L))
    case = SY.local_case("dominant", 77, [L] * len(probes), window=W, num_q_heads=2,
                         num_kv_heads=1, rope=False, fp8=fp8)
    case.q[:, 1, :] = case.q[:, 0, :]                 # equal heads in the group
    for s, j in enumerate(probes):
        qd = case.q[s, 0].astype(np.float64)
        idx = np.nonzero((case.tok_seq == s) & (case.tok_pos == j))[0][0]
        case.k[idx, 0] = (200.0 * qd / np.linalg.norm(qd)).astype(np.float32)
    return case, probes


@pytest.mark.parametrize("fp8", [False, True])
def test_dominant_key_probes(fp8):
    case, probes = dominant_case(fp8)
    _, out = run(case)
    for s, j in enumerate(probes):
        K, V = local_seq(case, s)
        want = V[j, 0].astype(np.float32)
        for h in range(2):
            got = out[s, h]
            assert np.array_equal(got, want), f"probe j*={j}: output is not V[j*] bit-for-bit"


def test_page_permutation_bitexact():
    a = SY.local_case("perm", 5, [700, 1500, 64, 2048], window=1024, num_q_heads=16,
                      num_kv_heads=8, rope=True)
    b = SY.local_case("perm", 5, [700, 1500, 64, 2048], window=1024, num_q_heads=16,
                      num_kv_heads=8, rope=True, extra_pages=37)   # other permutation, bigger pool
    assert not np.array_equal(a.seqs.page_table, b.seqs.page_table)
    b.q, b.k, b.v = a.q, a.k, a.v
    _, oa = run(a)
    _, ob = run(b)
    assert np.array_equal(oa, ob)


@pytest.mark.parametrize("fp8", [False, True])
def test_row_order_and_batch_bitexact(fp8):
    lens = [900, 3000, 1024, 33, 4100]
    base = SY.local_case("rows", 8, lens, window=1024, num_q_heads=16, num_kv_heads=8,
                         rope=True, fp8=fp8)
    _, o_all = run(base)
    # reversed order
    perm = np.arange(len(lens))[::-1]
    rev = SY.local_case("rows", 8, [lens[i] for i in perm], window=1024, num_q_heads=16,
                        num_kv_heads=8, rope=True, fp8=fp8)
    rev.q = base.q[perm]
    ks, vs, ts, ps = [], [], [], []
    for new_s, old_s in enumerate(perm):
        sel = base.tok_seq == old_s
        ks.append(base.k[sel]); vs.append(base.v[sel])
        ts.append(np.full(sel.sum(), new_s, np.int32)); ps.append(base.tok_pos[sel])
    rev.k, rev.v, rev.tok_seq, rev.tok_pos = (np.concatenate(ks), np.concatenate(vs),
                                              np.concatenate(ts), np.concatenate(ps))
    _, o_rev = run(rev)
    assert np.array_equal(o_rev, o_all[perm])
    # each row alone in its own call (other batch, other grid)
    for s in (1, 3):
        one = SY.local_case("one", 8, [lens[s]], window=1024, num_q_heads=16, num_kv_heads=8,
                            rope=True, fp8=fp8)
        sel = base.tok_seq == s
        one.q = base.q[s:s + 1]
        one.k, one.v = base.k[sel], base.v[sel]
        one.tok_seq = np.zeros(sel.sum(), np.int32)
        one.tok_pos = base.tok_pos[sel]
        _, o1 = run(one)
        assert np.array_equal(o1[0], o_all[s])


@pytest.mark.parametrize("fp8,hq", [(True, 16), (True, 32), (False, 32)])
def test_split_grouping_batch_invariant(fp8, hq):
    """A batch with more (sequence, KV head) splits than the device has CUs
    runs workgroups that each take 2 or 4 splits of a pair (e4m3 pages at
    group sizes 2 and 4, bf16 pages at group size 4); every row must equal,
    bit for bit, the same row computed alone (one split per workgroup)."""
    rng = np.random.default_rng(77 + hq + fp8)
    lens = [int(x) for x in rng.integers(2048, 8193, 48)]
    lens[5] = 2048          # aligned window
    lens[6] = 1030          # window that wraps a page
    lens[7] = 700           # shorter than the window: one split
    base = SY.local_case("grouped", 12, lens, window=1024, num_q_heads=hq, num_kv_heads=8,
                         rope=True, fp8=fp8, fill_window_only=True)
    _, o_all = run(base)
    for s in (0, 5, 6, 7, 47):
        one = SY.local_case("one", 12, [lens[s]], window=1024, num_q_heads=hq, num_kv_heads=8,
                            rope=True, fp8=fp8, fill_window_only=True)
        sel = base.tok_seq == s
        one.q = base.q[s:s + 1]
        one.k, one.v = base.k[sel], base.v[sel]
        one.tok_seq = np.zeros(sel.sum(), np.int32)
        one.tok_pos = base.tok_pos[sel]
        _, o1 = run(one)
        assert np.array_equal(o1[0], o_all[s]), f"row {s} (L={lens[s]}) differs from its solo call"


def test_repeat_determinism():
    case = SY.local_case("repeat", 9, [5000, 2000, 8000], window=1024, num_q_heads=16,
                         num_kv_heads=8, rope=True)
    dc, o1 = run(case)
    o2 = RT.attend(dc).cpu().numpy()
    o3 = RT.attend(dc).cpu().numpy()
    assert np.array_equal(o1, o2) and np.array_equal(o1, o3)
    # one workspace over many calls: the split counters and the partials'
    # call tags carry over from call to call
    ws = RT.Workspace()
    for _ in range(6):
        assert np.array_equal(o1, RT.attend(dc, ws=ws).cpu().numpy())


def test_workspace_shared_across_shapes():
    # calls of two shapes (more sequences, so more split counters, in the
    # second) take turns on one workspace: each result equals the one from a
    # fresh workspace, bit for bit
    ca = SY.local_case("ws_a", 21, [5000, 2000, 8000], window=1024, num_q_heads=16, num_kv_heads=8, rope=True)
    cb = SY.local_case("ws_b", 22, [3000, 7000, 1500, 6000, 4000, 2500, 8000], window=1024, num_q_heads=16,
                       num_kv_heads=8, rope=True)
    da, oa = run(ca)
    db, ob = run(cb)
    ws = RT.Workspace()
    for _ in range(3):
        assert np.array_equal(oa, RT.attend(da, ws=ws).cpu().numpy())
        assert np.array_equal(ob, RT.attend(db, ws=ws).cpu().numpy())


# ------------------------------------------------------------- append ------
def pool_bytes(dc):
    torch.cuda.synchronize()
    return dc.pool.buf.cpu().numpy()


@pytest.mark.parametrize("fp8", [False, True])
def test_append_local_rotated(fp8):
    case = SY.local_case("append", 12, [100, 37, 530], window=1024, num_q_heads=4, num_kv_heads=2,
                         rope=True, fp8=fp8, extra_pages=3)
    dc = RT.upload_local(case)
    pb = pool_bytes(dc)
    eb = 1 if fp8 else 2
    dec = OC.e4m3_decode if fp8 else OC.bf16_decode
    for s in range(case.seqs.S):
        L = int(case.seqs.lens[s])
        Kc, Vc = OP.local_codes(pb, case.seqs.page_table[s], L, 2, eb)
        K, V = local_seq(case, s)
        # V is stored exactly as rounded; K within one step of the stored grid
        assert np.array_equal(dec(Vc), V)
        gk = dec(Kc)
        if fp8:
            # one e4m3 step is 2^-3 relative; a one-ulp bf16 difference in the
            # rotated value can move a tie
            tol = np.maximum(np.abs(K), 2.0 ** -6) * 2.0 ** -3
        else:
            tol = np.maximum(np.abs(K), 2.0 ** -126) * 2.0 ** -7
        assert np.all(np.abs(gk - K) <= tol + 1e-30)
        frac_exact = np.mean(gk == K)
        assert frac_exact > 0.95, frac_exact
    # pages outside the table stay untouched
    used = set(case.seqs.page_table[case.seqs.page_table >= 0].tolist())
    per_page = dc.pool.page_bytes
    for p in range(case.seqs.num_pages):
        if p not in used:
            assert np.all(pb[p * per_page:(p + 1) * per_page] == 0xFF)


def test_e4m3_encode_all_bf16_patterns():
    """Every bf16 bit pattern through the GPU store: e4m3 code must equal the
    oracle's nearest-even saturating encode of that bf16 value."""
    pat = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = OC.bf16_decode(pat)                      # incl. NaN and inf patterns
    case = SY.local_case("enc", 3, [256], window=256, num_q_heads=1, num_kv_heads=1, rope=False,
                         fp8=True)
    case.k = vals.reshape(256, 1, 256).astype(np.float32)
    case.v = vals.reshape(256, 1, 256).astype(np.float32)[::-1].copy()
    dc = RT.upload_local(case)
    pb = pool_bytes(dc)
    Kc, Vc = OP.local_codes(pb, case.seqs.page_table[0], 256, 1, 1)
    for got, src in ((Kc, case.k), (Vc, case.v)):
        want = OC.e4m3_encode(src.astype(np.float64))
        nan = np.isnan(src)
        assert np.array_equal(got[~nan], want[~nan])
        assert np.all((got[nan] & 0x7F) == 0x7F)


def test_e4m3_decode_all_codes():
    """Window 1: each output is its own token's V, i.e. the decoded e4m3 value
    of each of the 256 codes (one per dim) -- the GPU's fp8 -> bf16 path."""
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    vals = OC.e4m3_decode(codes)
    vals = np.where(np.isnan(vals), 1.0, vals)      # keep the output finite
    case = SY.local_case("dec", 4, [16], window=1, num_q_heads=1, num_kv_heads=1, rope=False, fp8=True)
    case.v[:] = 0
    case.v[15, 0, :] = vals.astype(np.float32)
    _, out = run(case)
    assert np.array_equal(out[0, 0], vals.astype(np.float32))


@pytest.mark.parametrize("fp8,rope", [(False, True), (True, True), (False, False), (True, False)])
def test_fused_append_matches_separate(fp8, rope):
    """Appending each row's token inside the attention call writes the same
    pool bytes and gives the same outputs, bit for bit, as gw_kv_append
    followed by attention."""
    lens = [1, 17, 700, 1500, 4096, 16, 1024, 1041]
    case = SY.local_case("fused", 55, lens, window=1024, num_q_heads=16, num_kv_heads=8, rope=rope,
                         fp8=fp8, q_scale=0.5, kv_scale=0.5)
    dc_sep = RT.upload_local(case)
    out_sep = RT.attend(dc_sep).cpu().numpy()

    last = np.array([np.nonzero((case.tok_seq == s) & (case.tok_pos == L - 1))[0][0]
                     for s, L in enumerate(lens)])
    keep = np.ones(case.tok_seq.shape[0], bool)
    keep[last] = False
    import copy
    c2 = copy.copy(case)
    c2.k, c2.v, c2.tok_seq, c2.tok_pos = case.k[keep], case.v[keep], case.tok_seq[keep], case.tok_pos[keep]
    dc_f = RT.upload_local(c2)
    k_new = RT.to_bf16_dev(case.k[last])
    v_new = RT.to_bf16_dev(case.v[last])
    rope_t = RT.rope_tables(int(max(lens)), 256, 256, RT.LOCAL_THETA) if rope else None
    out_f = RT.attend(dc_f, k_new=k_new, v_new=v_new, rope=rope_t).cpu().numpy()
    torch.cuda.synchronize()
    assert torch.equal(dc_f.pool.buf, dc_sep.pool.buf), "pool bytes differ"
    assert np.array_equal(out_f, out_sep)
    # the call is repeatable: the same step again gives the same result
    out_f2 = RT.attend(dc_f, k_new=k_new, v_new=v_new, rope=rope_t).cpu().numpy()
    assert np.array_equal(out_f2, out_sep)
