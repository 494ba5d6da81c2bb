"""Global family on the GPU: append of the compressed and full records and
paged MQA decode attention (head dim 512, one tied KV head) against the CPU
oracle, plus the bit-exact gates (compressed == full, page placement, row
order, dominant-key probes).  Tolerances: max abs 1e-2, mean abs 1e-3."""

import numpy as np
import pytest
import torch

from oracle import codecs as OC
from oracle import pool as OP
from oracle import rope as OR
from paged_hybrid_kv_amd import runtime as RT, synth as SY

from .oracle_side import compare, global_seq, oracle_out

pytestmark = pytest.mark.gpu


def run(case, compressed=True):
    dc = RT.upload_global(case, compressed=compressed)
    out = RT.attend(dc)
    torch.cuda.synchronize()
    return dc, out.cpu().numpy()


def check(case, out, label, seqs=None):
    ref = oracle_out(case, seqs)
    worst = 0.0
    for s, r in ref.items():
        mx, _, _ = compare(out[s:s + 1], r, f"{label} seq {s}")
        worst = max(worst, mx)
    return worst


@pytest.mark.parametrize("rope", [False, True])
def test_small_global(rope):
    lens = [1, 2, 16, 17, 31, 32, 33, 63, 64, 65, 700, 4097]
    case = SY.global_case("small", 30, lens, num_q_heads=32, rope=rope)
    _, oc = run(case, True)
    _, of = run(case, False)
    assert np.array_equal(oc, of), "compressed and full records differ"
    mx = check(case, oc, f"small rope={rope}")
    print(f"global small rope={rope} max abs err {mx:.2e}", flush=True)


def test_sixteen_heads():
    case = SY.global_case("h16", 31, [5, 300, 2000], num_q_heads=16, rope=True)
    _, out = run(case)
    check(case, out, "Hq=16")


def test_global_full_size():
    """8 slots x 131072 tokens: every slot compared bit-exactly between the two
    records; two slots against the oracle."""
    case = SY.global_tied()
    dc, oc = run(case, True)
    del dc
    torch.cuda.empty_cache()
    dcf, of = run(case, False)
    del dcf
    torch.cuda.empty_cache()
    assert np.array_equal(oc, of), "compressed and full records differ at 131072 tokens"
    mx = check(case, oc, "global_tied", seqs=[0, 5])
    print(f"global_tied (2 of 8 slots) max abs err {mx:.2e}", flush=True)


def test_dominant_key_probes():
    L = 100
    probes = [0, 1, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 95, 96, 98, 99]
    case = SY.global_case("dominant", 33, [L] * len(probes), num_q_heads=32, rope=False)
    case.q[:] = case.q[:, :1, :]                      # all heads equal
    for s, j in enumerate(probes):
        qd = case.q[s, 0].astype(np.float64)
        idx = np.nonzero((case.tok_seq == s) & (case.tok_pos == j))[0][0]
        case.v[idx] = (200.0 * qd / np.linalg.norm(qd)).astype(np.float32)   # K = V (tied)
    for compressed in (True, False):
        _, out = run(case, compressed)
        for s, j in enumerate(probes):
            _, V = global_seq(case, s)
            want = V[j, 0].astype(np.float32)
            for h in range(32):
                assert np.array_equal(out[s, h], want), f"probe j*={j} head {h}"


def test_page_permutation_and_row_order_bitexact():
    lens = [3000, 129, 4500, 64]
    a = SY.global_case("perm", 34, lens, rope=True)
    b = SY.global_case("perm", 34, lens, rope=True, extra_pages=11)
    assert not np.array_equal(a.seqs.page_table, b.seqs.page_table)
    b.q, b.v = a.q, a.v
    _, oa = run(a)
    _, ob = run(b)
    assert np.array_equal(oa, ob)
    # reverse the rows
    perm = np.arange(len(lens))[::-1]
    r = SY.global_case("perm", 35, [lens[i] for i in perm], rope=True)
    r.q = a.q[perm]
    vs, ts, ps = [], [], []
    for new_s, old_s in enumerate(perm):
        sel = a.tok_seq == old_s
        vs.append(a.v[sel]); ts.append(np.full(sel.sum(), new_s, np.int32)); ps.append(a.tok_pos[sel])
    r.v, r.tok_seq, r.tok_pos = np.concatenate(vs), np.concatenate(ts), np.concatenate(ps)
    _, orr = run(r)
    assert np.array_equal(orr, oa[perm])


def test_repeat_determinism():
    case = SY.global_case("repeat", 36, [20000, 9000], rope=True)
    dc, o1 = run(case)
    o2 = RT.attend(dc).cpu().numpy()
    assert np.array_equal(o1, o2)


def test_reduce_schedules_bitexact():
    """The cross-split reduce has two schedules of the same arithmetic, picked
    from the call's largest split count: a row of 29 splits alone takes the
    sequential one, beside a row of 63 splits the parallel one.  The row's
    result must not depend on which (nor on the row's place in the batch);
    the 63-split row is checked against the oracle."""
    both = SY.global_case("sched", 37, [20000, 9000], rope=True)
    alone = SY.global_case("sched", 38, [9000], rope=True)
    sel = both.tok_seq == 1
    alone.q = both.q[1:2]
    alone.v, alone.tok_pos = both.v[sel], both.tok_pos[sel]
    alone.tok_seq = np.zeros(int(sel.sum()), both.tok_seq.dtype)
    for compressed in (True, False):
        _, ob = run(both, compressed)
        _, oa = run(alone, compressed)
        assert np.array_equal(ob[1:2], oa), f"schedules differ (compressed={compressed})"
    mx = check(both, ob, "reduce schedules", seqs=[0])
    print(f"63-split row max abs err {mx:.2e}", flush=True)


@pytest.mark.parametrize("compressed", [True, False])
def test_append_global(compressed):
    case = SY.global_case("append", 37, [40, 17, 300], rope=True, extra_pages=2)
    dc = RT.upload_global(case, compressed=compressed)
    torch.cuda.synchronize()
    pb = dc.pool.buf.cpu().numpy()
    for s in range(case.seqs.S):
        L = int(case.seqs.lens[s])
        A, B = OP.global_codes(pb, case.seqs.page_table[s], L, compressed)
        sel = case.tok_seq == s
        v = OC.bf16_round(case.v[sel].astype(np.float64))
        k_rot = OC.bf16_round(OR.rotate_global(v, case.tok_pos[sel])[:, :128])
        if compressed:
            Vg, Kr = OC.bf16_decode(A), OC.bf16_decode(B)
        else:
            Kg, Vg = OC.bf16_decode(A), OC.bf16_decode(B)
            assert np.array_equal(Kg[:, 128:], v[:, 128:])
            Kr = Kg[:, :128]
        assert np.array_equal(Vg, v)
        tol = np.maximum(np.abs(k_rot), 2.0 ** -126) * 2.0 ** -7
        assert np.all(np.abs(Kr - k_rot) <= tol)
        assert np.mean(Kr == k_rot) > 0.95


def k_before_rotation(case):
    """The K a k_norm model hands over: the stored bf16 V times w_k.  Both
    carry at most 8 significant bits, so the fp32 product is exact and the
    bf16 cast on upload rounds it once, as the oracle side does."""
    vb = torch.from_numpy(case.v).to(torch.bfloat16).float().numpy()
    return vb * case.w_k


@pytest.mark.parametrize("rope", [False, True])
def test_norm_weighted_k(rope):
    """K = V * w_k before rotation (a per-dim norm weight on K): the append
    takes that K for the rotated quarter and the caller folds w_k into q's
    dims 128..511; the output matches the oracle's attention over the true K,
    and both records agree bit for bit."""
    lens = [1, 33, 700, 4097]
    case = SY.global_case("knorm", 38, lens, num_q_heads=32, rope=rope, k_norm=True)
    k_raw = k_before_rotation(case)
    q_fold = case.q.copy()
    q_fold[..., 128:] *= case.w_k[128:]
    outs = []
    for compressed in (True, False):
        dc = RT.upload_global(case, compressed=compressed, k_raw=k_raw, q=q_fold)
        outs.append(RT.attend(dc).cpu().numpy())
        del dc
    assert np.array_equal(outs[0], outs[1]), "compressed and full records differ"
    mx = check(case, outs[0], f"k_norm rope={rope}")
    print(f"global k_norm rope={rope} max abs err {mx:.2e}", flush=True)
    # the tied store of the same V gives another answer: the weight matters
    tied = SY.global_case("knorm", 38, lens, num_q_heads=32, rope=rope)
    _, ot = run(tied)
    assert np.abs(ot - outs[0]).max() > 1e-2


@pytest.mark.parametrize("mixed", [False, True])
def test_norm_weighted_k_in_call(mixed):
    """The query rows' own tokens appended inside the attention call, with K
    before rotation given apart from V (k_new: a norm weight on K), in decode
    rows and, in a mixed call, prompt rows too: the outputs equal, bit for
    bit, those of the same tokens appended beforehand by gw_kv_append with
    k_raw, in both records, and match the oracle's attention over the true K."""
    lens = [700, 4097, 33, 2000]
    q_len = [1, 1, 1, 1] if not mixed else [1, 24, 1, 7]
    case = SY.global_case("knorm_call", 41, lens, num_q_heads=32, rope=True, k_norm=True, q_len=q_len)
    k_raw = k_before_rotation(case)
    q_fold = case.q.copy()
    q_fold[..., 128:] *= case.w_k[128:]
    # the rows' tokens: the last q_len of each sequence, in row order
    rows = []
    for s, (L, ql) in enumerate(zip(lens, q_len)):
        for pos in range(L - ql, L):
            rows.append(int(np.nonzero((case.tok_seq == s) & (case.tok_pos == pos))[0][0]))
    rows = np.array(rows)
    keep = np.ones(case.tok_seq.shape[0], bool)
    keep[rows] = False
    import copy
    pre = copy.copy(case)
    pre.tok_seq, pre.tok_pos, pre.v = case.tok_seq[keep], case.tok_pos[keep], case.v[keep]
    rope = RT.rope_tables(max(lens), 128, 512, RT.GLOBAL_THETA)
    outs = {}
    for compressed in (True, False):
        dc = RT.upload_global(case, compressed=compressed, k_raw=k_raw, q=q_fold)
        outs[compressed, "before"] = RT.attend(dc).cpu().numpy()
        del dc
        dc = RT.upload_global(pre, compressed=compressed, k_raw=k_raw[keep], q=q_fold)
        outs[compressed, "in_call"] = RT.attend(dc, k_new=RT.to_bf16_dev(k_raw[rows]),
                                                v_new=RT.to_bf16_dev(case.v[rows]), rope=rope).cpu().numpy()
        del dc
        torch.cuda.empty_cache()
    for compressed in (True, False):
        assert np.array_equal(outs[compressed, "in_call"], outs[compressed, "before"]), \
            f"in-call append with k_new differs from gw_kv_append with k_raw (compressed={compressed})"
    assert np.array_equal(outs[True, "in_call"], outs[False, "in_call"]), "compressed and full records differ"
    ref = oracle_out(case)
    qi = case.q_indptr
    mx = max(compare(outs[True, "in_call"][qi[s]:qi[s + 1]], r, f"k_norm in call mixed={mixed} seq {s}")[0]
             for s, r in ref.items())
    print(f"global k_norm in-call mixed={mixed}: max abs err {mx:.2e}", flush=True)


def test_append_global_norm_weighted_k():
    """The record's rotated quarter comes from k_raw, V from v, in both layouts."""
    case = SY.global_case("append_knorm", 39, [40, 300], rope=True, k_norm=True)
    k_raw = k_before_rotation(case)
    for compressed in (True, False):
        dc = RT.upload_global(case, compressed=compressed, k_raw=k_raw)
        torch.cuda.synchronize()
        pb = dc.pool.buf.cpu().numpy()
        for s in range(case.seqs.S):
            L = int(case.seqs.lens[s])
            A, B = OP.global_codes(pb, case.seqs.page_table[s], L, compressed)
            sel = case.tok_seq == s
            v = OC.bf16_round(case.v[sel].astype(np.float64))
            k_pre = OC.bf16_round(v * case.w_k.astype(np.float64))
            k_rot = OC.bf16_round(OR.rotate_global(k_pre, case.tok_pos[sel])[:, :128])
            if compressed:
                Vg, Kr = OC.bf16_decode(A), OC.bf16_decode(B)
            else:
                Kg, Vg = OC.bf16_decode(A), OC.bf16_decode(B)
                assert np.array_equal(Kg[:, 128:], v[:, 128:])
                Kr = Kg[:, :128]
            assert np.array_equal(Vg, v)
            tol = np.maximum(np.abs(k_rot), 2.0 ** -126) * 2.0 ** -7
            assert np.all(np.abs(Kr - k_rot) <= tol)
            assert np.mean(Kr == k_rot) > 0.95
        del dc
