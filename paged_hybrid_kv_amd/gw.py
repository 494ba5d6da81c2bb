"""ctypes binding of libgw.so (include/gw.h), same names as the C ABI.

Argument marshalling only: tensors become device pointers, None becomes
NULL, the stream defaults to torch's current stream.  Every step of the
path runs in the library's HIP kernels; there is no fallback, and a missing
library raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgw.so")

GW_OK = 0
GW_ERR_INVALID_ARG = -1
GW_ERR_UNSUPPORTED = -2
GW_ERR_GEOMETRY = -3
GW_ERR_WORKSPACE = -4
GW_ERR_HIP = -5
GW_ERR_REFUSED = -6

GW_FAMILY_LOCAL = 1
GW_FAMILY_GLOBAL_COMPRESSED = 2
GW_FAMILY_GLOBAL_FULL = 3

GW_KV_BF16 = 1
GW_KV_E4M3 = 2

EXPORTS = ("gw_version", "gw_last_error", "gw_pool_page_bytes", "gw_rope_table", "gw_kv_append",
           "gw_attn_workspace_bytes", "gw_decode_attn_local", "gw_decode_attn_local_noalloc",
           "gw_decode_attn_global",
           "gw_alloc_create", "gw_alloc_destroy", "gw_alloc_admit", "gw_alloc_extend", "gw_alloc_release",
           "gw_alloc_tables", "gw_alloc_stats", "gw_copy_pages")


class GwError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code
        self.message = message


class gw_pool_desc(ctypes.Structure):
    _fields_ = [
        ("family", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rot_dim", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("base", ctypes.c_void_p),
    ]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def lib():
    """Load libgw.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with paged_hybrid_kv_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.gw_version.restype = ctypes.c_char_p
        L.gw_version.argtypes = []
        L.gw_last_error.restype = ctypes.c_char_p
        L.gw_last_error.argtypes = []
        L.gw_pool_page_bytes.restype = ctypes.c_int64
        L.gw_pool_page_bytes.argtypes = [ctypes.POINTER(gw_pool_desc)]
        L.gw_rope_table.restype = ctypes.c_int
        L.gw_rope_table.argtypes = [_P, _P, _I, _I, _I, ctypes.c_double, _P]
        L.gw_kv_append.restype = ctypes.c_int
        L.gw_kv_append.argtypes = [ctypes.POINTER(gw_pool_desc), _P, _P, _P, _P, _I, _P, _I, _P, _P, _P]
        L.gw_attn_workspace_bytes.restype = ctypes.c_size_t
        L.gw_attn_workspace_bytes.argtypes = [_I] * 8
        L.gw_decode_attn_local.restype = ctypes.c_int
        L.gw_decode_attn_local.argtypes = [ctypes.POINTER(gw_pool_desc), _P, _I, _P, _P, _P, _P, _P, _P,
                                           _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P, _P,
                                           ctypes.c_size_t, _P]
        L.gw_decode_attn_local_noalloc.restype = ctypes.c_int
        L.gw_decode_attn_local_noalloc.argtypes = [ctypes.POINTER(gw_pool_desc), _P, _I, _P, _P, _P, _P, _P,
                                                   _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P, _P]
        L.gw_decode_attn_global.restype = ctypes.c_int
        L.gw_decode_attn_global.argtypes = [ctypes.POINTER(gw_pool_desc), _P, _I, _P, _P, _P, _P, _P, _P, _P,
                                            _I, _I, _I, _I, _I, ctypes.c_float, _P, _P, ctypes.c_size_t,
                                            _P]
        L.gw_alloc_create.restype = ctypes.c_int
        L.gw_alloc_create.argtypes = [_I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_void_p)]
        L.gw_alloc_destroy.restype = ctypes.c_int
        L.gw_alloc_destroy.argtypes = [_P]
        L.gw_alloc_admit.restype = ctypes.c_int
        L.gw_alloc_admit.argtypes = [_P, _I, _I, ctypes.POINTER(ctypes.c_int32)]
        L.gw_alloc_extend.restype = ctypes.c_int
        L.gw_alloc_extend.argtypes = [_P, _I, _I, _I]
        L.gw_alloc_release.restype = ctypes.c_int
        L.gw_alloc_release.argtypes = [_P, _I]
        L.gw_alloc_tables.restype = ctypes.c_int
        L.gw_alloc_tables.argtypes = [_P, _P, _I, _P, _I, _P]
        L.gw_alloc_stats.restype = ctypes.c_int
        L.gw_alloc_stats.argtypes = [_P, _P]
        L.gw_copy_pages.restype = ctypes.c_int
        L.gw_copy_pages.argtypes = [ctypes.POINTER(gw_pool_desc), ctypes.POINTER(gw_pool_desc), _P, _P, _I, _P]
        _lib = L
    return _lib


def _ptr(x):
    """None -> NULL; int -> that address; tensor -> its data pointer."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(rc: int):
    if rc != GW_OK:
        raise GwError(rc, lib().gw_last_error().decode())


def gw_version() -> str:
    return lib().gw_version().decode()


def gw_last_error() -> str:
    return lib().gw_last_error().decode()


def gw_pool_page_bytes(desc: gw_pool_desc) -> int:
    r = lib().gw_pool_page_bytes(ctypes.byref(desc))
    if r < 0:
        _check(int(r))
    return int(r)


def gw_rope_table(cos_out, sin_out, max_pos, rot_dim, head_dim, theta, stream=None):
    _check(lib().gw_rope_table(_ptr(cos_out), _ptr(sin_out), max_pos, rot_dim, head_dim, theta,
                               _stream(stream)))


def gw_kv_append(desc: gw_pool_desc, k_raw, v, seq_idx, pos, n_tok, page_table, pt_stride,
                 rope_cos=None, rope_sin=None, stream=None):
    _check(lib().gw_kv_append(ctypes.byref(desc), _ptr(k_raw), _ptr(v), _ptr(seq_idx), _ptr(pos),
                              n_tok, _ptr(page_table), pt_stride, _ptr(rope_cos), _ptr(rope_sin),
                              _stream(stream)))


def gw_attn_workspace_bytes(family, num_seqs, num_rows, num_q_heads, head_dim, max_seq_len,
                            window, max_q_len) -> int:
    return int(lib().gw_attn_workspace_bytes(family, num_seqs, num_rows, num_q_heads, head_dim,
                                             max_seq_len, window, max_q_len))


def gw_decode_attn_local(desc: gw_pool_desc, q, num_q_heads, k_new, v_new, rope_cos, rope_sin,
                         q_indptr, seq_lens, page_table, pt_stride, num_seqs, num_rows, max_q_len,
                         max_seq_len, window, scale, out, workspace, workspace_bytes, stream=None):
    _check(lib().gw_decode_attn_local(ctypes.byref(desc), _ptr(q), num_q_heads, _ptr(k_new),
                                      _ptr(v_new), _ptr(rope_cos), _ptr(rope_sin), _ptr(q_indptr),
                                      _ptr(seq_lens), _ptr(page_table), pt_stride, num_seqs,
                                      num_rows, max_q_len, max_seq_len, window, scale, _ptr(out),
                                      _ptr(workspace), workspace_bytes, _stream(stream)))


def gw_decode_attn_local_noalloc(desc: gw_pool_desc, q, num_q_heads, k_new, v_new, rope_cos, rope_sin,
                                 q_indptr, seq_lens, page_table, pt_stride, num_seqs, num_rows, max_q_len,
                                 max_seq_len, window, scale, out, stream=None):
    _check(lib().gw_decode_attn_local_noalloc(ctypes.byref(desc), _ptr(q), num_q_heads, _ptr(k_new),
                                              _ptr(v_new), _ptr(rope_cos), _ptr(rope_sin), _ptr(q_indptr),
                                              _ptr(seq_lens), _ptr(page_table), pt_stride, num_seqs,
                                              num_rows, max_q_len, max_seq_len, window, scale, _ptr(out),
                                              _stream(stream)))


def gw_decode_attn_global(desc: gw_pool_desc, q, num_q_heads, k_new, v_new, rope_cos, rope_sin, q_indptr,
                          seq_lens, page_table, pt_stride, num_seqs, num_rows, max_q_len, max_seq_len,
                          scale, out, workspace, workspace_bytes, stream=None):
    _check(lib().gw_decode_attn_global(ctypes.byref(desc), _ptr(q), num_q_heads, _ptr(k_new), _ptr(v_new),
                                       _ptr(rope_cos), _ptr(rope_sin), _ptr(q_indptr),
                                       _ptr(seq_lens), _ptr(page_table), pt_stride, num_seqs,
                                       num_rows, max_q_len, max_seq_len, scale, _ptr(out),
                                       _ptr(workspace), workspace_bytes, _stream(stream)))


# ------------------------------------------------------- pool lifecycle --
class PageAllocator:
    """gw_alloc_*: the two families' page ids and the decode slots (host
    only).  Tables come back as numpy int32 arrays."""

    def __init__(self, slots, max_context, window, local_pages, global_pages):
        h = ctypes.c_void_p()
        _check(lib().gw_alloc_create(slots, max_context, window, local_pages, global_pages, ctypes.byref(h)))
        self.h = h.value
        self.slots, self.max_context = slots, max_context
        self.pages_per_slot = (max_context + 15) // 16

    def close(self):
        if self.h:
            lib().gw_alloc_destroy(self.h)
            self.h = None

    __del__ = close

    def admit(self, total_tokens, max_step_rows):
        """Slot index, or -1 to wait; raises GwError(GW_ERR_REFUSED) when refused."""
        slot = ctypes.c_int32(-1)
        _check(lib().gw_alloc_admit(self.h, total_tokens, max_step_rows, ctypes.byref(slot)))
        return slot.value

    def extend(self, slot, new_len, first_query_pos):
        _check(lib().gw_alloc_extend(self.h, slot, new_len, first_query_pos))

    def release(self, slot):
        _check(lib().gw_alloc_release(self.h, slot))

    def tables(self):
        import numpy as np
        n = self.pages_per_slot
        lpt = np.empty((self.slots, n), dtype=np.int32)
        gpt = np.empty((self.slots, n), dtype=np.int32)
        lens = np.empty(self.slots, dtype=np.int32)
        _check(lib().gw_alloc_tables(self.h, lpt.ctypes.data, n, gpt.ctypes.data, n, lens.ctypes.data))
        return lpt, gpt, lens

    def stats(self):
        """(free local, free global, reserved local, reserved global, active, slots)"""
        import numpy as np
        st = np.empty(6, dtype=np.int32)
        _check(lib().gw_alloc_stats(self.h, st.ctypes.data))
        return tuple(int(x) for x in st)


def gw_copy_pages(dst: gw_pool_desc, src: gw_pool_desc, dst_pages, src_pages, n, stream=None):
    _check(lib().gw_copy_pages(ctypes.byref(dst), ctypes.byref(src), _ptr(dst_pages), _ptr(src_pages), n,
                               _stream(stream)))
