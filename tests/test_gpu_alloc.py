"""Pool lifecycle on the GPU: gw_copy_pages bit for bit, and decode
attention over page tables the host allocator produced (local pages before
the window freed, global pages all held) against the oracle."""

import dataclasses

import numpy as np
import pytest
import torch

from paged_hybrid_kv_amd import gw, runtime as RT, synth as SY

from .oracle_side import compare, oracle_out

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("family,dt", [(gw.GW_FAMILY_LOCAL, gw.GW_KV_BF16),
                                       (gw.GW_FAMILY_GLOBAL_COMPRESSED, gw.GW_KV_E4M3)])
def test_copy_pages_bitexact(family, dt):
    heads = 8 if family == gw.GW_FAMILY_LOCAL else 1
    src = RT.Pool(family, dt, 70, heads, fill_byte=0)
    dst = RT.Pool(family, dt, 90, heads, fill_byte=0x5A)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    src.buf.copy_(torch.randint(0, 256, src.buf.shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8))
    rng = np.random.default_rng(8)
    s_ids = rng.choice(70, 50, replace=False).astype(np.int32)
    d_ids = rng.choice(90, 50, replace=False).astype(np.int32)
    s_ids[7], d_ids[9] = 70, -1                 # out of range: those two pairs are skipped
    gw.gw_copy_pages(dst.desc, src.desc, RT.i32_dev(d_ids), RT.i32_dev(s_ids), 50)
    torch.cuda.synchronize()
    S = src.buf.cpu().numpy().reshape(70, -1)
    D = dst.buf.cpu().numpy().reshape(90, -1)
    done = set()
    for i, (d, s) in enumerate(zip(d_ids, s_ids)):
        if i in (7, 9):
            continue
        assert np.array_equal(D[d], S[s]), i
        done.add(int(d))
    for d in set(range(90)) - done:
        assert (D[d] == 0x5A).all(), d


def test_decode_over_allocator_tables():
    """Four requests grown one token per step by the allocator; the local
    case reads its K/V through the allocator's local table (front of the
    window freed), the global case through its global table."""
    lens = [1500, 3000, 700, 4097]
    A = gw.PageAllocator(4, 8192, 1024, 4 * 65 + 7, 4 * 512)
    for s, L in enumerate(lens):
        assert A.admit(8192, 1) == s
        for n in range(1, L + 1):
            A.extend(s, n, n - 1)
    lpt, gpt, alens = A.tables()
    assert list(alens) == lens

    loc = SY.local_case("alloc local", 50, lens, window=1024, num_q_heads=16, num_kv_heads=8, q_scale=0.5,
                        kv_scale=0.5, rope=True, window_only_pages=True, fill_window_only=True)
    w = loc.seqs.page_table.shape[1]
    assert np.array_equal(lpt[:, :w] >= 0, loc.seqs.page_table >= 0)
    assert (lpt[:, w:] < 0).all()
    loc.seqs = dataclasses.replace(loc.seqs, page_table=np.ascontiguousarray(lpt[:, :w]), num_pages=4 * 65 + 7)
    out = RT.attend(RT.upload_local(loc)).cpu().numpy()
    for s, r in oracle_out(loc).items():
        compare(out[s:s + 1], r, f"local over allocator table, seq {s}")

    glb = SY.global_case("alloc global", 51, lens, num_q_heads=32, rope=True)
    w = glb.seqs.page_table.shape[1]
    assert np.array_equal(gpt[:, :w] >= 0, glb.seqs.page_table >= 0)
    glb.seqs = dataclasses.replace(glb.seqs, page_table=np.ascontiguousarray(gpt[:, :w]), num_pages=4 * 512)
    out = RT.attend(RT.upload_global(glb)).cpu().numpy()
    for s, r in oracle_out(glb).items():
        compare(out[s:s + 1], r, f"global over allocator table, seq {s}")
