"""Device-side plumbing around the C ABI: pools, rotary tables, uploads and
calls for whole workloads.  Memory comes from torch; every computation is a
libgw.so kernel call.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import gw
from .synth import GlobalCase, LocalCase, PAGE

LOCAL_THETA = 1.0e4
GLOBAL_THETA = 1.0e6


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("paged_hybrid_kv_amd needs a ROCm GPU (MI355X); none is visible")
    gw.lib()


def to_bf16_dev(x: np.ndarray, device="cuda") -> torch.Tensor:
    """fp32 host draws -> bf16 device tensor (torch's nearest-even cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device).to(torch.bfloat16)


def i32_dev(x, device="cuda") -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32)).to(device)


class Pool:
    """One layer's paged pool: a device byte buffer plus its descriptor."""

    def __init__(self, family: int, kv_dtype: int, num_pages: int, num_kv_heads: int = 1,
                 rot_dim: int | None = None, device="cuda", fill_byte: int | None = None):
        head_dim = 256 if family == gw.GW_FAMILY_LOCAL else 512
        if rot_dim is None:
            rot_dim = 256 if family == gw.GW_FAMILY_LOCAL else 128
        self.desc = gw.gw_pool_desc(family, kv_dtype, PAGE, num_kv_heads, head_dim, rot_dim,
                                    num_pages, None)
        self.page_bytes = gw.gw_pool_page_bytes(self.desc)
        n = num_pages * self.page_bytes
        if fill_byte is None:
            self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        else:
            self.buf = torch.full((n,), fill_byte, dtype=torch.uint8, device=device)
        self.desc.base = self.buf.data_ptr()
        self.family, self.kv_dtype = family, kv_dtype
        self.num_pages, self.num_kv_heads, self.head_dim, self.rot_dim = num_pages, num_kv_heads, head_dim, rot_dim


_rope_cache: dict = {}


def rope_tables(max_pos: int, rot_dim: int, head_dim: int, theta: float, device="cuda"):
    """(cos, sin) fp32 [max_pos][rot_dim/2] filled by gw_rope_table (cached)."""
    key = (max_pos, rot_dim, head_dim, theta, str(device))
    t = _rope_cache.get(key)
    if t is None or t[0].shape[0] < max_pos:
        cos = torch.empty(max_pos * (rot_dim // 2), dtype=torch.float32, device=device)
        sin = torch.empty_like(cos)
        gw.gw_rope_table(cos, sin, max_pos, rot_dim, head_dim, theta)
        t = (cos, sin)
        _rope_cache[key] = t
    return t


def identity_rope_tables(max_pos: int, rot_dim: int, device="cuda"):
    """cos = 1, sin = 0: the rotation leaves K as given (exact in fp32)."""
    n = max_pos * (rot_dim // 2)
    return (torch.ones(n, dtype=torch.float32, device=device),
            torch.zeros(n, dtype=torch.float32, device=device))


@dataclass
class DeviceCase:
    """A workload uploaded to the GPU and appended into its pool."""
    pool: Pool
    q: torch.Tensor
    q_indptr: torch.Tensor | None
    seq_lens: torch.Tensor
    page_table: torch.Tensor
    pt_stride: int
    num_seqs: int
    num_rows: int
    max_q_len: int
    max_seq_len: int
    num_q_heads: int
    scale: float
    window: int | None


def upload_local(case: LocalCase, device="cuda", fill_byte: int | None = 0xFF,
                 append_chunk: int = 1 << 16) -> DeviceCase:
    """Pool, tables and q on the device; K/V appended with gw_kv_append.

    The pool starts as all-ones bytes (NaN in bf16 and e4m3), so a read of a
    slot the workload never wrote poisons the result.
    """
    require_gpu()
    dt = gw.GW_KV_E4M3 if case.fp8 else gw.GW_KV_BF16
    rot = 256 if case.rope else 0
    pool = Pool(gw.GW_FAMILY_LOCAL, dt, case.seqs.num_pages, case.num_kv_heads, rot, device, fill_byte)
    pt = i32_dev(case.seqs.page_table, device)
    stride = case.seqs.page_table.shape[1]
    max_len = int(case.seqs.lens.max())
    cos = sin = None
    if case.rope:
        cos, sin = rope_tables(max_len, 256, 256, LOCAL_THETA, device)
    n = case.tok_seq.shape[0]
    for c0 in range(0, n, append_chunk):
        c1 = min(n, c0 + append_chunk)
        k = to_bf16_dev(case.k[c0:c1], device)
        v = to_bf16_dev(case.v[c0:c1], device)
        gw.gw_kv_append(pool.desc, k, v, i32_dev(case.tok_seq[c0:c1], device),
                        i32_dev(case.tok_pos[c0:c1], device), c1 - c0, pt, stride, cos, sin)
    q = to_bf16_dev(case.q, device)
    single = bool((case.q_len == 1).all())
    return DeviceCase(pool=pool, q=q, q_indptr=None if single else i32_dev(case.q_indptr, device),
                      seq_lens=i32_dev(case.seqs.lens, device), page_table=pt, pt_stride=stride,
                      num_seqs=case.seqs.S, num_rows=int(case.q_len.sum()),
                      max_q_len=int(case.q_len.max()), max_seq_len=max_len,
                      num_q_heads=case.num_q_heads, scale=case.scale, window=case.window)


def upload_global(case: GlobalCase, compressed: bool = True, device="cuda",
                  fill_byte: int | None = 0xFF, append_chunk: int = 1 << 17,
                  k_raw: np.ndarray | None = None, q: np.ndarray | None = None) -> DeviceCase:
    """Append the case's tokens into a fresh pool and stage its queries.
    k_raw [n_tok][512] (fp32, sent as bf16), when given, is K before rotation
    for the tokens (its first 128 dims make the rotated quarter); q, when
    given, replaces the case's queries (the caller's own q for that K)."""
    require_gpu()
    fam = gw.GW_FAMILY_GLOBAL_COMPRESSED if compressed else gw.GW_FAMILY_GLOBAL_FULL
    pool = Pool(fam, gw.GW_KV_E4M3 if case.fp8 else gw.GW_KV_BF16, case.seqs.num_pages, 1, 128, device, fill_byte)
    pt = i32_dev(case.seqs.page_table, device)
    stride = case.seqs.page_table.shape[1]
    max_len = int(case.seqs.lens.max())
    if case.rope:
        cos, sin = rope_tables(max_len, 128, 512, GLOBAL_THETA, device)
    else:
        cos, sin = identity_rope_tables(max_len, 128, device)
    n = case.tok_seq.shape[0]
    for c0 in range(0, n, append_chunk):
        c1 = min(n, c0 + append_chunk)
        v = to_bf16_dev(case.v[c0:c1], device)
        k = None if k_raw is None else to_bf16_dev(k_raw[c0:c1], device)
        gw.gw_kv_append(pool.desc, k, v, i32_dev(case.tok_seq[c0:c1], device),
                        i32_dev(case.tok_pos[c0:c1], device), c1 - c0, pt, stride, cos, sin)
    q = to_bf16_dev(case.q if q is None else q, device)
    single = bool((case.q_len == 1).all())
    return DeviceCase(pool=pool, q=q, q_indptr=None if single else i32_dev(case.q_indptr, device),
                      seq_lens=i32_dev(case.seqs.lens, device), page_table=pt, pt_stride=stride,
                      num_seqs=case.seqs.S, num_rows=int(case.q_len.sum()),
                      max_q_len=int(case.q_len.max()), max_seq_len=max_len,
                      num_q_heads=case.num_q_heads, scale=case.scale, window=None)


class Workspace:
    """Grow-only device workspace, 256-byte aligned, zero-filled when
    (re)allocated.  The library leaves it ready for the next call of the same
    shape; where its split counters and call epochs sit depends on the shape,
    so a call of another shape (another `key`: the arguments the size was
    asked for with) gets it zero-filled again first."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None
        self.key = None

    def get(self, nbytes: int, key=None):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes + 256:
            self.buf = torch.zeros(nbytes + 256, dtype=torch.uint8, device=self.device)
        elif key != self.key:
            self.buf.zero_()
        self.key = key
        addr = self.buf.data_ptr()
        aligned = (addr + 255) // 256 * 256
        return aligned, nbytes


def attend(dc: DeviceCase, out: torch.Tensor | None = None, ws: Workspace | None = None,
           stream=None, k_new=None, v_new=None, rope=None) -> torch.Tensor:
    """One attention call over an uploaded workload; returns fp32 [rows][Hq][D].

    k_new/v_new (+ rope = (cos, sin)): append each row's own token in the call.
    """
    local = dc.pool.family == gw.GW_FAMILY_LOCAL
    D = dc.pool.head_dim
    if out is None:
        out = torch.empty((dc.num_rows, dc.num_q_heads, D), dtype=torch.float32, device=dc.q.device)
    ws = ws or Workspace(dc.q.device)
    shape = (dc.pool.family, dc.num_seqs, dc.num_rows, dc.num_q_heads, D, dc.max_seq_len,
             dc.window if local else 0, dc.max_q_len)
    need = gw.gw_attn_workspace_bytes(*shape)
    wptr, wbytes = ws.get(need, (shape, dc.pool.num_kv_heads))
    cos, sin = rope if rope is not None else (None, None)
    if local:
        gw.gw_decode_attn_local(dc.pool.desc, dc.q, dc.num_q_heads, k_new, v_new, cos, sin,
                                dc.q_indptr, dc.seq_lens,
                                dc.page_table, dc.pt_stride, dc.num_seqs, dc.num_rows, dc.max_q_len,
                                dc.max_seq_len, dc.window, dc.scale, out, wptr, wbytes, stream)
    else:
        gw.gw_decode_attn_global(dc.pool.desc, dc.q, dc.num_q_heads, k_new, v_new, cos, sin,
                                 dc.q_indptr, dc.seq_lens,
                                 dc.page_table, dc.pt_stride, dc.num_seqs, dc.num_rows, dc.max_q_len,
                                 dc.max_seq_len, dc.scale, out, wptr, wbytes, stream)
    return out
