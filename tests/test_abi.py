"""The C-ABI library loads, exports every symbol include/gw.h declares, and
rejects invalid calls on the host before any HIP call (so these run with no
GPU).  Error conventions follow pegainfer PR #1012: a width outside the
enum is unrepresentable, a refused combination carries a fixed message, and
a failure names the entry point that ran."""

import ctypes
import os
import re

import pytest

from paged_hybrid_kv_amd import gw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gw.h")

pytestmark = pytest.mark.skipif(not os.path.exists(gw.LIB_PATH), reason="libgw.so not built")

FAKE = 0x1000   # non-null stand-in address; never dereferenced by a rejected call


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gw_[a-z_0-9]+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(gw.EXPORTS)
    L = gw.lib()
    for n in names:
        assert hasattr(L, n), n


def test_version():
    assert "gfx950" in gw.gw_version()


def desc(family=gw.GW_FAMILY_LOCAL, dt=gw.GW_KV_BF16, page=16, heads=8, dim=None, rot=None, pages=4,
         base=FAKE):
    if dim is None:
        dim = 256 if family == gw.GW_FAMILY_LOCAL else 512
    if rot is None:
        rot = 256 if family == gw.GW_FAMILY_LOCAL else 128
    if family != gw.GW_FAMILY_LOCAL and heads == 8:
        heads = 1
    return gw.gw_pool_desc(family, dt, page, heads, dim, rot, pages, base)


def test_page_bytes():
    assert gw.gw_pool_page_bytes(desc()) == 16 * 2 * 8 * 256 * 2
    assert gw.gw_pool_page_bytes(desc(dt=gw.GW_KV_E4M3)) == 16 * 2 * 8 * 256
    comp = gw.gw_pool_page_bytes(desc(gw.GW_FAMILY_GLOBAL_COMPRESSED))
    full = gw.gw_pool_page_bytes(desc(gw.GW_FAMILY_GLOBAL_FULL))
    assert (comp, full) == (20480, 32768) and comp / full == 0.625
    comp8 = gw.gw_pool_page_bytes(desc(gw.GW_FAMILY_GLOBAL_COMPRESSED, dt=gw.GW_KV_E4M3))
    full8 = gw.gw_pool_page_bytes(desc(gw.GW_FAMILY_GLOBAL_FULL, dt=gw.GW_KV_E4M3))
    assert (comp8, full8) == (10240, 16384)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(family=0), gw.GW_ERR_INVALID_ARG, "unknown family"),
    (dict(dt=0), gw.GW_ERR_INVALID_ARG, "unknown kv_dtype"),
    (dict(dt=3), gw.GW_ERR_INVALID_ARG, "unknown kv_dtype"),
    (dict(page=32), gw.GW_ERR_GEOMETRY, "page_size"),
    (dict(dim=128), gw.GW_ERR_GEOMETRY, "head_dim"),
    (dict(rot=64), gw.GW_ERR_GEOMETRY, "rot_dim"),
    (dict(heads=0), gw.GW_ERR_GEOMETRY, "num_kv_heads"),
    (dict(family=gw.GW_FAMILY_GLOBAL_FULL, heads=2), gw.GW_ERR_GEOMETRY, "num_kv_heads"),
    (dict(family=gw.GW_FAMILY_GLOBAL_FULL, rot=512), gw.GW_ERR_GEOMETRY, "rot_dim"),
])
def test_page_bytes_rejects(kw, code, frag):
    with pytest.raises(gw.GwError) as e:
        gw.gw_pool_page_bytes(desc(**kw))
    assert e.value.code == code
    assert e.value.message.startswith("gw_pool_page_bytes: ")
    assert frag in e.value.message


def append(d, k=FAKE, v=FAKE, n=4, stride=8, cos=FAKE, sin=FAKE):
    gw.gw_kv_append(d, k, v, FAKE, FAKE, n, FAKE, stride, cos, sin)


@pytest.mark.parametrize("call,code,frag", [
    (lambda: append(desc(base=None)), gw.GW_ERR_INVALID_ARG, "base is null"),
    (lambda: append(desc(pages=0)), gw.GW_ERR_INVALID_ARG, "num_pages"),
    (lambda: append(desc(), n=-1), gw.GW_ERR_INVALID_ARG, "n_tok"),
    (lambda: append(desc(), cos=None), gw.GW_ERR_INVALID_ARG, "both"),
    (lambda: append(desc(), cos=None, sin=None), gw.GW_ERR_INVALID_ARG, "needs rotary tables"),
    (lambda: append(desc(rot=0)), gw.GW_ERR_INVALID_ARG, "takes no rotary tables"),
    (lambda: append(desc(family=gw.GW_FAMILY_GLOBAL_FULL), k=None, cos=None, sin=None),
     gw.GW_ERR_INVALID_ARG, "needs rotary tables"),
    (lambda: append(desc(), k=None), gw.GW_ERR_INVALID_ARG, "k_raw is null"),
    (lambda: append(desc(), stride=0), gw.GW_ERR_INVALID_ARG, "pt_stride"),
])
def test_append_rejects(call, code, frag):
    with pytest.raises(gw.GwError) as e:
        call()
    assert e.value.code == code
    assert e.value.message.startswith("gw_kv_append: ")
    assert frag in e.value.message


def test_append_zero_tokens_is_noop():
    append(desc(), n=0)   # returns GW_OK without touching the GPU


def local(d=None, q=FAKE, hq=16, kn=None, vn=None, cos=None, sin=None, indptr=None, lens=FAKE, pt=FAKE,
          stride=512, S=4, rows=4, mql=1, msl=8192, win=1024, scale=0.0625, out=FAKE, ws=FAKE,
          wsb=1 << 30):
    gw.gw_decode_attn_local(d or desc(), q, hq, kn, vn, cos, sin, indptr, lens, pt, stride, S, rows, mql,
                            msl, win, scale, out, ws, wsb, None)


def glob(d=None, q=FAKE, hq=32, kn=None, vn=None, cos=None, sin=None, indptr=None, lens=FAKE, pt=FAKE,
         stride=8192, S=4, rows=4, mql=1, msl=131072, scale=0.044, out=FAKE, ws=FAKE, wsb=1 << 30):
    gw.gw_decode_attn_global(d or desc(gw.GW_FAMILY_GLOBAL_COMPRESSED), q, hq, kn, vn, cos, sin, indptr, lens,
                             pt, stride, S, rows, mql, msl, scale, out, ws, wsb, None)


@pytest.mark.parametrize("call,code,frag", [
    (lambda: local(win=0), gw.GW_ERR_INVALID_ARG, "window"),
    (lambda: local(hq=12), gw.GW_ERR_GEOMETRY, "multiple"),
    (lambda: local(hq=64), gw.GW_ERR_UNSUPPORTED, "group size 8"),
    (lambda: local(d=desc(gw.GW_FAMILY_GLOBAL_FULL)), gw.GW_ERR_INVALID_ARG, "not GW_FAMILY_LOCAL"),
    (lambda: local(rows=5), gw.GW_ERR_INVALID_ARG, "num_rows"),
    (lambda: local(mql=2), gw.GW_ERR_INVALID_ARG, "max_q_len"),
    (lambda: local(stride=10), gw.GW_ERR_INVALID_ARG, "pt_stride"),
    (lambda: local(q=None), gw.GW_ERR_INVALID_ARG, "null"),
    (lambda: local(out=None), gw.GW_ERR_INVALID_ARG, "null"),
    (lambda: local(scale=float("nan")), gw.GW_ERR_INVALID_ARG, "scale"),
    (lambda: local(S=-1), gw.GW_ERR_INVALID_ARG, "num_seqs"),
    (lambda: local(wsb=16), gw.GW_ERR_WORKSPACE, "workspace"),
    (lambda: local(ws=None), gw.GW_ERR_INVALID_ARG, "workspace is null"),
    (lambda: local(ws=FAKE + 8), gw.GW_ERR_INVALID_ARG, "aligned"),
    (lambda: local(d=desc(dt=gw.GW_KV_BF16, page=8)), gw.GW_ERR_GEOMETRY, "page_size"),
    (lambda: local(kn=FAKE), gw.GW_ERR_INVALID_ARG, "k_new and v_new"),
    (lambda: local(kn=FAKE, vn=FAKE), gw.GW_ERR_INVALID_ARG, "needs rotary tables"),
    (lambda: local(kn=FAKE, vn=FAKE, cos=FAKE), gw.GW_ERR_INVALID_ARG, "both"),
    (lambda: local(d=desc(rot=0), kn=FAKE, vn=FAKE, cos=FAKE, sin=FAKE), gw.GW_ERR_INVALID_ARG,
     "takes no rotary tables"),
    # grids past 2^31 - 1 workgroups are refused before any launch: the
    # decode rows' (split, KV head, sequence) grid ...
    (lambda: local(d=desc(heads=65535), hq=65535, S=65535, rows=65535, stride=512, wsb=1 << 62),
     gw.GW_ERR_UNSUPPORTED, "decode workgroups"),
    # ... the same grid's workgroups past the decode items, which append the
    # prompt rows' own tokens (page item x two KV heads)
    (lambda: local(d=desc(heads=32768), hq=32768, S=4096, rows=2 ** 31 - 1, indptr=FAKE, mql=8192, win=1,
                   kn=FAKE, vn=FAKE, cos=FAKE, sin=FAKE, ws=None, wsb=0),
     gw.GW_ERR_UNSUPPORTED, "append workgroups"),
    # ... and the prompt rows' (row block, KV head) grid
    (lambda: local(d=desc(heads=32768), hq=32768, S=65535, rows=2 ** 31 - 1, indptr=FAKE, mql=8192, win=1,
                   ws=None, wsb=0),
     gw.GW_ERR_UNSUPPORTED, "prompt-row workgroups"),
])
def test_local_rejects(call, code, frag):
    with pytest.raises(gw.GwError) as e:
        call()
    assert e.value.code == code
    assert e.value.message.startswith("gw_decode_attn_local: ")
    assert frag in e.value.message


@pytest.mark.parametrize("call,code,frag", [
    (lambda: glob(hq=8), gw.GW_ERR_UNSUPPORTED, "num_q_heads"),
    (lambda: glob(d=desc()), gw.GW_ERR_INVALID_ARG, "not a global family"),
    (lambda: glob(wsb=0), gw.GW_ERR_WORKSPACE, "workspace"),
    (lambda: glob(msl=0), gw.GW_ERR_INVALID_ARG, "max_seq_len"),
    (lambda: glob(vn=FAKE), gw.GW_ERR_INVALID_ARG, "rotary tables"),
    (lambda: glob(kn=FAKE), gw.GW_ERR_INVALID_ARG, "k_new is set but v_new is null"),
])
def test_global_rejects(call, code, frag):
    with pytest.raises(gw.GwError) as e:
        call()
    assert e.value.code == code
    assert e.value.message.startswith("gw_decode_attn_global: ")
    assert frag in e.value.message


def test_local_noalloc_rejects():
    # the same host checks as the workspace entry point, named after the
    # entry point that ran, and a plan too large for the library's scratch
    # array refused before any HIP call
    def noalloc(**kw):
        a = dict(d=desc(), q=FAKE, hq=16, lens=FAKE, pt=FAKE, stride=512, S=4, rows=4, mql=1, msl=8192,
                 win=1024, scale=0.0625, out=FAKE)
        a.update(kw)
        gw.gw_decode_attn_local_noalloc(a["d"], a["q"], a["hq"], None, None, None, None, None, a["lens"],
                                        a["pt"], a["stride"], a["S"], a["rows"], a["mql"], a["msl"], a["win"],
                                        a["scale"], a["out"])
    for kw, code, frag in ((dict(win=0), gw.GW_ERR_INVALID_ARG, "window"),
                           (dict(hq=64), gw.GW_ERR_UNSUPPORTED, "group size 8"),
                           (dict(S=65535, rows=65535), gw.GW_ERR_WORKSPACE, "scratch")):
        with pytest.raises(gw.GwError) as e:
            noalloc(**kw)
        assert e.value.code == code
        assert e.value.message.startswith("gw_decode_attn_local_noalloc: ")
        assert frag in e.value.message
    noalloc(S=0, rows=0)   # empty batch: no-op, no GPU call


def test_empty_batches_are_noops():
    local(S=0, rows=0, ws=None, wsb=0)
    glob(S=0, rows=0, ws=None, wsb=0)


def test_workspace_plan():
    # one window of 1024 tokens is 64 pages of work -> at most 4 splits of 16
    # pages (the size query assumes query-group size 4, the most splits);
    # local partials are 8-byte (value, tag) pairs
    ws = gw.gw_attn_workspace_bytes(gw.GW_FAMILY_LOCAL, 16, 16, 16, 256, 8192, 1024, 1)
    assert ws >= 16 * 16 * 4 * 258 * 8
    assert gw.gw_attn_workspace_bytes(gw.GW_FAMILY_LOCAL, 1, 1, 2, 256, 64, 32, 1) == 0
    wg = gw.gw_attn_workspace_bytes(gw.GW_FAMILY_GLOBAL_COMPRESSED, 8, 8, 32, 512, 131072, 0, 1)
    assert wg >= 8 * 32 * 64 * 514 * 4
    assert gw.gw_attn_workspace_bytes(gw.GW_FAMILY_GLOBAL_FULL, 1, 1, 32, 512, 256, 0, 1) == 0


def test_workspace_rezeroed_for_another_shape():
    # the library leaves a workspace ready for the next call of the same
    # shape only: the host-side holder zero-fills it again when the shape
    # (the arguments its size was asked for with) changes
    import torch
    from paged_hybrid_kv_amd import runtime as RT
    ws = RT.Workspace("cpu")
    ws.get(4096, "a")
    ws.buf.fill_(7)
    ws.get(4096, "a")
    assert int(ws.buf.sum()) == 7 * ws.buf.numel()   # same shape: kept
    ws.get(1024, "b")
    assert int(ws.buf.count_nonzero()) == 0          # another shape: zero-filled
    assert ws.get(0, "c") == (None, 0)


def test_error_message_is_thread_local_and_cleared():
    with pytest.raises(gw.GwError):
        local(win=0)
    assert gw.gw_last_error().startswith("gw_decode_attn_local")
    assert gw.gw_pool_page_bytes(desc()) > 0
    assert gw.gw_last_error() == ""


def test_copy_pages_rejects():
    a, b = desc(), desc(gw.GW_FAMILY_GLOBAL_FULL)
    for d, sd, n, code, frag in ((a, b, 1, gw.GW_ERR_GEOMETRY, "differ"),
                                 (a, desc(dt=gw.GW_KV_E4M3), 1, gw.GW_ERR_GEOMETRY, "differ"),
                                 (a, a, -1, gw.GW_ERR_INVALID_ARG, "n -1")):
        with pytest.raises(gw.GwError) as e:
            gw.gw_copy_pages(d, sd, FAKE, FAKE, n)
        assert e.value.code == code and frag in e.value.message
    gw.gw_copy_pages(a, a, FAKE, FAKE, 0)      # n == 0: no-op, no GPU call
