"""Prompt rows (sequences with q_len > 1) on the GPU: the same attention
entry points, mixed with decode rows, against the CPU oracle, plus the
bit-exact gates: prompt rows give the same bits in a mixed call as alone,
compressed == full for the global family, dominant-key probes at the causal
and window edges, and the in-call append of every row's token equal to a
standalone append.  Tolerances: max abs 1e-2, mean abs 1e-3."""

import copy

import numpy as np
import pytest
import torch

from oracle import codecs as OC
from paged_hybrid_kv_amd import gw, runtime as RT, synth as SY

from .oracle_side import compare, global_seq, local_seq, oracle_out

pytestmark = pytest.mark.gpu


def rows(out, case, s):
    qi = case.q_indptr
    return out[qi[s]:qi[s + 1]]


def check(case, out, label):
    ref = oracle_out(case)
    worst = 0.0
    for s, r in ref.items():
        mx, _, _ = compare(rows(out, case, s), r, f"{label} seq {s}")
        worst = max(worst, mx)
    return worst


def run_local(case):
    dc = RT.upload_local(case)
    out = RT.attend(dc)
    torch.cuda.synchronize()
    return dc, out.cpu().numpy()


def run_global(case, compressed=True):
    dc = RT.upload_global(case, compressed=compressed)
    out = RT.attend(dc)
    torch.cuda.synchronize()
    return dc, out.cpu().numpy()


# ------------------------------------------------------------------ local --
@pytest.mark.parametrize("fp8", [False, True])
def test_local_prompt_rows_mixed(fp8):
    # decode rows and prompt rows in one call; a prompt with prior context
    # (a chunk of a longer prompt) and one without
    lens = [600, 1500, 5, 64, 3000, 700, 2]
    q_len = [512, 100, 5, 1, 1, 33, 2]
    case = SY.local_case("prefill", 61, lens, window=1024, num_q_heads=16, num_kv_heads=8,
                         q_len=q_len, rope=True, fp8=fp8, q_scale=0.5, kv_scale=0.5)
    _, out = run_local(case)
    mx = check(case, out, f"local prompt rows fp8={fp8}")
    print(f"local prompt rows fp8={fp8}: max abs err {mx:.2e}", flush=True)


@pytest.mark.parametrize("G,Hkv", [(1, 2), (2, 3), (4, 2)])
def test_local_prompt_group_sizes(G, Hkv):
    case = SY.local_case("prefill groups", 62 + G, [300, 47, 1100], window=256, num_q_heads=G * Hkv,
                         num_kv_heads=Hkv, q_len=[300, 20, 90], rope=False)
    _, out = run_local(case)
    check(case, out, f"prompt G={G}")


@pytest.mark.parametrize("W", [1, 16, 37, 100])
def test_local_prompt_window_narrower_than_prompt(W):
    # the window slides inside the prompt: row r sees [r - W + 1, r]
    case = SY.local_case(f"prefill W={W}", 70 + W, [400, 129, 17], window=W, num_q_heads=4,
                         num_kv_heads=2, q_len=[400, 64, 17], rope=False, kv_scale=0.5, q_scale=0.5)
    _, out = run_local(case)
    check(case, out, f"prompt window {W}")


@pytest.mark.parametrize("fp8", [False, True])
def test_local_prompt_dominant_keys(fp8):
    """Every prompt row has the same query u; K[j*] = 200 u for one j*.  A row
    whose window holds j* must return V[j*] bit for bit; the others must
    match the oracle (which gives them zero weight on j*)."""
    L, W = 160, 48
    probes = [0, 15, 16, 47, 48, 95, 100, 159]
    case = SY.local_case("prefill dominant", 80, [L] * len(probes), window=W, num_q_heads=2,
                         num_kv_heads=1, q_len=[L] * len(probes), rope=False, fp8=fp8)
    u = case.q[0, 0].copy()
    case.q[:] = u
    for s, j in enumerate(probes):
        idx = np.nonzero((case.tok_seq == s) & (case.tok_pos == j))[0][0]
        case.k[idx, 0] = (200.0 * u / np.linalg.norm(u.astype(np.float64))).astype(np.float32)
    _, out = run_local(case)
    for s, j in enumerate(probes):
        _, V = local_seq(case, s)
        want = V[j, 0].astype(np.float32)
        got = rows(out, case, s)
        for r in range(L):
            if max(0, r - W + 1) <= j <= r:
                for h in range(2):
                    assert np.array_equal(got[r, h], want), f"probe j*={j} row {r} head {h}"
    check(case, out, "prefill dominant")


def test_local_mixed_equals_separate_calls():
    """Rows of a call depend only on their own sequence: the prompt rows of a
    mixed call equal those of a call with the prompts alone, and the decode
    rows equal a decode-only call, bit for bit."""
    lens = [900, 300, 2000, 512]
    q_len = [1, 300, 1, 200]
    mixed = SY.local_case("mixed", 90, lens, window=1024, num_q_heads=16, num_kv_heads=8, q_len=q_len,
                          rope=True)
    _, o_mixed = run_local(mixed)
    for keep in ([1, 3], [0, 2]):
        part = SY.local_case("mixed", 90, [lens[i] for i in keep], window=1024, num_q_heads=16,
                             num_kv_heads=8, q_len=[q_len[i] for i in keep], rope=True)
        qs, ks, vs, ts, ps = [], [], [], [], []
        for new_s, old_s in enumerate(keep):
            qs.append(rows(mixed.q, mixed, old_s))
            sel = mixed.tok_seq == old_s
            ks.append(mixed.k[sel]); vs.append(mixed.v[sel])
            ts.append(np.full(sel.sum(), new_s, np.int32)); ps.append(mixed.tok_pos[sel])
        part.q = np.concatenate(qs)
        part.k, part.v = np.concatenate(ks), np.concatenate(vs)
        part.tok_seq, part.tok_pos = np.concatenate(ts), np.concatenate(ps)
        _, o_part = run_local(part)
        for new_s, old_s in enumerate(keep):
            assert np.array_equal(rows(o_part, part, new_s), rows(o_mixed, mixed, old_s)), (keep, old_s)


@pytest.mark.parametrize("fp8", [False, True])
def test_local_in_call_append_mixed(fp8):
    """k_new / v_new for every row of a mixed call: the pool ends up as with
    gw_kv_append of those tokens, and the outputs are the same bits."""
    lens = [700, 40, 1500, 17, 30]        # prompts starting on, before and after a page edge
    q_len = [1, 40, 1, 9, 13]
    case = SY.local_case("append mixed", 95, lens, window=1024, num_q_heads=16, num_kv_heads=8,
                         q_len=q_len, rope=True, fp8=fp8, q_scale=0.5, kv_scale=0.5)
    dc_sep = RT.upload_local(case)
    out_sep = RT.attend(dc_sep).cpu().numpy()
    is_row = np.zeros(case.tok_seq.shape[0], bool)
    for s, (L, ql) in enumerate(zip(lens, q_len)):
        is_row |= (case.tok_seq == s) & (case.tok_pos >= L - ql)
    c2 = copy.copy(case)
    c2.k, c2.v = case.k[~is_row], case.v[~is_row]
    c2.tok_seq, c2.tok_pos = case.tok_seq[~is_row], case.tok_pos[~is_row]
    dc_f = RT.upload_local(c2)
    k_new, v_new = RT.to_bf16_dev(case.k[is_row]), RT.to_bf16_dev(case.v[is_row])
    rope_t = RT.rope_tables(int(max(lens)), 256, 256, RT.LOCAL_THETA)
    out_f = RT.attend(dc_f, k_new=k_new, v_new=v_new, rope=rope_t).cpu().numpy()
    torch.cuda.synchronize()
    assert torch.equal(dc_f.pool.buf, dc_sep.pool.buf), "pool bytes differ"
    assert np.array_equal(out_f, out_sep)


# ----------------------------------------------------------------- global --
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("hq", [16, 32])
def test_global_prompt_rows_mixed(hq, fp8):
    lens = [700, 300, 33, 4100, 2]
    q_len = [300, 1, 33, 1, 2]
    case = SY.global_case("prefill global", 100 + hq, lens, num_q_heads=hq, q_len=q_len, rope=True, fp8=fp8)
    _, oc = run_global(case, True)
    _, of = run_global(case, False)
    assert np.array_equal(oc, of), "compressed and full records differ"
    mx = check(case, oc, f"global prompt rows hq={hq} fp8={fp8}")
    print(f"global prompt rows hq={hq} fp8={fp8}: max abs err {mx:.2e}", flush=True)


@pytest.mark.parametrize("fp8", [False, True])
def test_global_prompt_dominant_keys(fp8):
    L = 100
    probes = [0, 15, 16, 31, 50, 99]
    case = SY.global_case("prefill global dominant", 110, [L] * len(probes), num_q_heads=32,
                          q_len=[L] * len(probes), rope=False, fp8=fp8)
    u = case.q[0, 0].copy()
    case.q[:] = u
    for s, j in enumerate(probes):
        idx = np.nonzero((case.tok_seq == s) & (case.tok_pos == j))[0][0]
        case.v[idx] = (200.0 * u / np.linalg.norm(u.astype(np.float64))).astype(np.float32)
    for compressed in (True, False):
        _, out = run_global(case, compressed)
        for s, j in enumerate(probes):
            _, V = global_seq(case, s)
            want = V[j, 0].astype(np.float32)
            got = rows(out, case, s)
            for r in range(j, L):
                assert np.array_equal(got[r, 0], want) and np.array_equal(got[r, 31], want), \
                    f"probe j*={j} row {r}"
        check(case, out, f"global dominant compressed={compressed} fp8={fp8}")


@pytest.mark.parametrize("fp8", [False, True])
def test_global_in_call_append_mixed(fp8):
    lens = [300, 45, 2000, 30]
    q_len = [1, 45, 1, 13]
    case = SY.global_case("global append mixed", 115, lens, q_len=q_len, rope=True, fp8=fp8)
    for compressed in (True, False):
        dc_sep = RT.upload_global(case, compressed=compressed)
        out_sep = RT.attend(dc_sep).cpu().numpy()
        is_row = np.zeros(case.tok_seq.shape[0], bool)
        for s, (L, ql) in enumerate(zip(lens, q_len)):
            is_row |= (case.tok_seq == s) & (case.tok_pos >= L - ql)
        c2 = copy.copy(case)
        c2.v, c2.tok_seq, c2.tok_pos = case.v[~is_row], case.tok_seq[~is_row], case.tok_pos[~is_row]
        dc_f = RT.upload_global(c2, compressed=compressed)
        rope_t = RT.rope_tables(int(max(lens)), 128, 512, RT.GLOBAL_THETA)
        out_f = RT.attend(dc_f, v_new=RT.to_bf16_dev(case.v[is_row]), rope=rope_t).cpu().numpy()
        torch.cuda.synchronize()
        assert torch.equal(dc_f.pool.buf, dc_sep.pool.buf), f"pool bytes differ (compressed={compressed})"
        assert np.array_equal(out_f, out_sep)


def test_global_decode_in_call_append_one_row_per_sequence():
    """v_new without q_indptr: each row's token is its sequence's last."""
    lens = [77, 1000, 16]
    case = SY.global_case("global append decode", 116, lens, rope=True)
    dc_sep = RT.upload_global(case)
    out_sep = RT.attend(dc_sep).cpu().numpy()
    last = np.array([np.nonzero((case.tok_seq == s) & (case.tok_pos == L - 1))[0][0] for s, L in enumerate(lens)])
    keep = np.ones(case.tok_seq.shape[0], bool)
    keep[last] = False
    c2 = copy.copy(case)
    c2.v, c2.tok_seq, c2.tok_pos = case.v[keep], case.tok_seq[keep], case.tok_pos[keep]
    dc_f = RT.upload_global(c2)
    rope_t = RT.rope_tables(int(max(lens)), 128, 512, RT.GLOBAL_THETA)
    out_f = RT.attend(dc_f, v_new=RT.to_bf16_dev(case.v[last]), rope=rope_t).cpu().numpy()
    torch.cuda.synchronize()
    assert torch.equal(dc_f.pool.buf, dc_sep.pool.buf)
    assert np.array_equal(out_f, out_sep)


# ------------------------------------------------------- many sequences --
def _many_seqs(seed, n=150, max_len=300):
    """n sequences (several 64-sequence chunks of the kernels' work scans),
    most of them decode rows, every fifth a prompt of 2..40 rows, some
    prompts starting mid-sequence."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(20, max_len, size=n)
    q_len = np.ones(n, dtype=np.int64)
    q_len[::5] = rng.integers(2, 41, size=q_len[::5].shape[0])
    q_len = np.minimum(q_len, lens)
    return lens, q_len


@pytest.mark.parametrize("n", [150, 300])
def test_local_many_sequences_in_call_append(n):
    """150 or 300 sequences mixing decode and prompt rows (300: past the 256
    sequences the prompt-row item lookup holds in registers), every row's
    token appended in the call: all rows against the oracle, and the pool
    and the outputs equal to a standalone append followed by the call."""
    lens, q_len = _many_seqs(120 if n == 150 else 125, n=n, max_len=300 if n == 150 else 160)
    case = SY.local_case("many local", 121, lens, window=64, num_q_heads=4, num_kv_heads=2,
                         q_len=q_len, rope=True, q_scale=0.5, kv_scale=0.5)
    dc_sep = RT.upload_local(case)
    out_sep = RT.attend(dc_sep).cpu().numpy()
    check(case, out_sep, "many local")
    is_row = np.zeros(case.tok_seq.shape[0], bool)
    for s, (L, ql) in enumerate(zip(lens, q_len)):
        is_row |= (case.tok_seq == s) & (case.tok_pos >= L - ql)
    c2 = copy.copy(case)
    c2.k, c2.v = case.k[~is_row], case.v[~is_row]
    c2.tok_seq, c2.tok_pos = case.tok_seq[~is_row], case.tok_pos[~is_row]
    dc_f = RT.upload_local(c2)
    k_new, v_new = RT.to_bf16_dev(case.k[is_row]), RT.to_bf16_dev(case.v[is_row])
    rope_t = RT.rope_tables(int(max(lens)), 256, 256, RT.LOCAL_THETA)
    out_f = RT.attend(dc_f, k_new=k_new, v_new=v_new, rope=rope_t).cpu().numpy()
    torch.cuda.synchronize()
    assert torch.equal(dc_f.pool.buf, dc_sep.pool.buf), "pool bytes differ"
    assert np.array_equal(out_f, out_sep)


@pytest.mark.parametrize("n", [150, 300])
@pytest.mark.parametrize("fp8", [False, True])
def test_global_many_sequences_in_call_append(fp8, n):
    lens, q_len = _many_seqs(130 if n == 150 else 135, n=n, max_len=400 if n == 150 else 200)
    case = SY.global_case("many global", 131, lens, num_q_heads=16, q_len=q_len, rope=True, fp8=fp8)
    dc_sep, out_sep = run_global(case)
    check(case, out_sep, "many global")
    is_row = np.zeros(case.tok_seq.shape[0], bool)
    for s, (L, ql) in enumerate(zip(lens, q_len)):
        is_row |= (case.tok_seq == s) & (case.tok_pos >= L - ql)
    c2 = copy.copy(case)
    c2.v = case.v[~is_row]
    c2.tok_seq, c2.tok_pos = case.tok_seq[~is_row], case.tok_pos[~is_row]
    dc_f = RT.upload_global(c2, compressed=True)
    v_new = RT.to_bf16_dev(case.v[is_row])
    rope_t = RT.rope_tables(int(max(lens)), 128, 512, RT.GLOBAL_THETA)
    out_f = RT.attend(dc_f, v_new=v_new, rope=rope_t).cpu().numpy()
    torch.cuda.synchronize()
    assert torch.equal(dc_f.pool.buf, dc_sep.pool.buf), "pool bytes differ"
    assert np.array_equal(out_f, out_sep)
