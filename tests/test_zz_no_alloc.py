"""The allocation-free local entry point (gw_decode_attn_local_noalloc,
whose split partials live in the library's own static scratch array) against
the workspace entry point (gw_decode_attn_local) on the same inputs: outputs
must be identical bit for bit.  Several calls in a row on the one array,
each smaller than the one before: the 16-slot bf16 window-1024 workload, a
3-sequence e4m3 call at group size 4 (another shape, so other counter and
partial positions), and a 2-sequence call with prompt rows and the rows'
tokens appended inside the call."""

import numpy as np
import pytest
import torch

from paged_hybrid_kv_amd import gw, runtime as RT, synth as SY

pytestmark = pytest.mark.gpu


def attend_noalloc(dc, out, k_new=None, v_new=None, rope=None):
    cos, sin = rope if rope is not None else (None, None)
    gw.gw_decode_attn_local_noalloc(dc.pool.desc, dc.q, dc.num_q_heads, k_new, v_new, cos, sin, dc.q_indptr,
                                    dc.seq_lens, dc.page_table, dc.pt_stride, dc.num_seqs, dc.num_rows,
                                    dc.max_q_len, dc.max_seq_len, dc.window, dc.scale, out)


def _cases():
    big = SY.local_bf16()
    small = SY.local_case("noalloc small", 61, [3000, 40, 1500], window=512, num_q_heads=32, num_kv_heads=8,
                          rope=True, fp8=True, q_scale=0.5, kv_scale=0.5)
    mixed = SY.local_case("noalloc mixed", 62, [700, 300], window=256, num_q_heads=16, num_kv_heads=8,
                          q_len=[1, 40], rope=True, q_scale=0.5, kv_scale=0.5)
    return big, small, mixed


def test_noalloc_matches_workspace_entry_point():
    big, small, mixed = _cases()
    for case in (big, small):
        print(f"noalloc: {case.name}, {case.seqs.S} sequences", flush=True)
        dc = RT.upload_local(case)
        ref = RT.attend(dc)
        out = torch.full_like(ref, float("nan"))
        attend_noalloc(dc, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{case.name}: outputs differ"
        del dc
    # prompt rows with each row's token appended in the call: both entry
    # points start from the same pool (the rows' tokens not yet written)
    print(f"noalloc: {mixed.name}, prompt rows appended in the call", flush=True)
    sel = np.ones(mixed.tok_seq.shape[0], bool)
    qi = mixed.q_indptr
    rows_pos = []
    for s, L in enumerate(mixed.seqs.lens):
        ql = qi[s + 1] - qi[s]
        for r in range(ql):
            p = int(L) - ql + r
            idx = np.nonzero((mixed.tok_seq == s) & (mixed.tok_pos == p))[0][0]
            sel[idx] = False
            rows_pos.append(idx)
    import copy
    base = copy.copy(mixed)
    base.k, base.v, base.tok_seq, base.tok_pos = mixed.k[sel], mixed.v[sel], mixed.tok_seq[sel], mixed.tok_pos[sel]
    k_new, v_new = RT.to_bf16_dev(mixed.k[rows_pos]), RT.to_bf16_dev(mixed.v[rows_pos])
    rope = RT.rope_tables(int(mixed.seqs.lens.max()), 256, 256, RT.LOCAL_THETA)
    dc_a, dc_b = RT.upload_local(base), RT.upload_local(base)
    ref = RT.attend(dc_a, k_new=k_new, v_new=v_new, rope=rope)
    out = torch.full_like(ref, float("nan"))
    attend_noalloc(dc_b, out, k_new=k_new, v_new=v_new, rope=rope)
    torch.cuda.synchronize()
    assert torch.equal(dc_a.pool.buf, dc_b.pool.buf), "pool bytes differ"
    assert torch.equal(out, ref), "outputs differ"
