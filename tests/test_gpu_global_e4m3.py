"""Global family in an e4m3 pool (codes of the bf16 record, scale 1.0) on
the GPU: append of both records, decode attention against the CPU oracle
over the decoded codes, compressed == full bit for bit, the in-call append
equal to a separate one, and the full-size 8 x 131072 workload on sampled
slots.  Tolerances: max abs 1e-2, mean abs 1e-3."""

import copy

import numpy as np
import pytest
import torch

from oracle import codecs as OC
from oracle import pool as OP
from oracle import rope as OR
from paged_hybrid_kv_amd import runtime as RT, synth as SY

from .oracle_side import compare, oracle_out

pytestmark = pytest.mark.gpu


def run(case, compressed=True):
    dc = RT.upload_global(case, compressed=compressed)
    out = RT.attend(dc)
    torch.cuda.synchronize()
    return dc, out.cpu().numpy()


def check(case, out, label, seqs=None):
    worst = 0.0
    for s, r in oracle_out(case, seqs).items():
        mx, _, _ = compare(out[s:s + 1], r, f"{label} seq {s}")
        worst = max(worst, mx)
    return worst


@pytest.mark.parametrize("hq", [32, 16])
@pytest.mark.parametrize("rope", [False, True])
def test_small_global_e4m3(rope, hq):
    lens = [1, 2, 16, 17, 31, 32, 33, 63, 64, 65, 700, 4097]
    case = SY.global_case("small_e4m3", 40, lens, num_q_heads=hq, rope=rope, fp8=True)
    _, oc = run(case, True)
    _, of = run(case, False)
    assert np.array_equal(oc, of), "compressed and full e4m3 records differ"
    mx = check(case, oc, f"e4m3 rope={rope} hq={hq}")
    print(f"global e4m3 rope={rope} hq={hq} max abs err {mx:.2e}", flush=True)


@pytest.mark.parametrize("compressed", [True, False])
def test_append_global_e4m3(compressed):
    case = SY.global_case("append_e4m3", 41, [40, 17, 300], rope=True, extra_pages=2, fp8=True)
    dc = RT.upload_global(case, compressed=compressed)
    torch.cuda.synchronize()
    pb = dc.pool.buf.cpu().numpy()
    for s in range(case.seqs.S):
        L = int(case.seqs.lens[s])
        A, B = OP.global_codes(pb, case.seqs.page_table[s], L, compressed, 1)
        sel = case.tok_seq == s
        v = OC.bf16_round(case.v[sel].astype(np.float64))
        k_rot = OC.bf16_round(OR.rotate_global(v, case.tok_pos[sel])[:, :128])
        if compressed:
            Vc, Kc = A, B
        else:
            Kc, Vc = A, B
            assert np.array_equal(Kc[:, 128:], Vc[:, 128:])
            Kc = Kc[:, :128]
        assert np.array_equal(Vc, OC.e4m3_encode(v))
        # the rotation is fp32 on the GPU: its bf16 value may sit one bf16 ulp
        # from the oracle's, which moves the e4m3 code by at most one step
        kd, kw = OC.e4m3_decode(Kc), OC.e4m3_decode(OC.e4m3_encode(k_rot))
        assert np.all(np.abs(kd - kw) <= np.maximum(np.abs(kw), 2.0 ** -6) * 2.0 ** -3)
        assert np.mean(Kc == OC.e4m3_encode(k_rot)) > 0.95


def test_in_call_append_e4m3():
    """v_new in the attention call writes the same pool bytes as the
    separate append and gives the same output bit for bit."""
    lens = [77, 1000, 16, 3001]
    case = SY.global_case("e4m3 append decode", 42, lens, rope=True, fp8=True)
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
    check(case, out_f, "e4m3 in-call append")


def test_repeat_and_page_permutation_e4m3():
    lens = [3000, 129, 4500, 64]
    a = SY.global_case("perm_e4m3", 43, lens, rope=True, fp8=True)
    b = SY.global_case("perm_e4m3", 43, lens, rope=True, extra_pages=11, fp8=True)
    assert not np.array_equal(a.seqs.page_table, b.seqs.page_table)
    b.q, b.v = a.q, a.v
    dca, oa = run(a)
    _, ob = run(b)
    assert np.array_equal(oa, ob)
    assert np.array_equal(RT.attend(dca).cpu().numpy(), oa)


def test_global_e4m3_full_size():
    """8 slots x 131072 tokens in the e4m3 compressed pool: two slots against
    the oracle."""
    case = SY.global_tied()
    case.fp8 = True
    dc, oc = run(case, True)
    del dc
    torch.cuda.empty_cache()
    mx = check(case, oc, "global_tied e4m3", seqs=[0, 5])
    print(f"global_tied e4m3 (2 of 8 slots) max abs err {mx:.2e}", flush=True)
