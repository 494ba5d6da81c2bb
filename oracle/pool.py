"""Paged KV pools: the documented element layouts, decoded back to contiguous
per-sequence K/V codes, and the per-family byte model.

Test infrastructure only (see ``oracle/__init__``).

pegainfer "Gemma 4" page, Scheduling: each attention family has its own paged
pool and budget; pages hold 16 tokens in both families; logical token t of a
sequence lives in physical page pt[t // 16] at slot t % 16.  Gewell post,
"the Why": the global family may store only V and the rotated quarter of K,
0.625x the bytes of a full K/V record.

The element order *inside* a page is this library's own (the pages do not fix
one); it is restated here from the public header, independently of the HIP
code, so that a test can read a pool the GPU wrote and compare it element by
element with what the oracle expects.

Local family, per page: [Hkv][K, V][block], block = 16 tokens x 256 dims.
  bf16 (2 B) K block: element ((k*16 + t)*4 + c)*8 + e  = K[t][64c + 8k + e]
                      k<8, t<16, c<4, e<8
  bf16 V block:       element ((u*64 + l)*4 + j)*2 + i  = V[2u + i][4l + j]
                      u<8, l<64, j<4, i<2
  e4m3 (1 B) K block: element ((k*16 + t)*4 + c)*16 + e = K[t][64c + 16k + e]
                      k<4, t<16, c<4, e<16
  e4m3 V block:       element ((u*64 + l)*4 + j)*4 + i  = V[4u + i][4l + j]
                      u<4, l<64, j<4, i<4
Global family, compressed page: V block [16][512] then K_rot block [16][128];
Global family, full page:       K block [16][512] then V block [16][512];
  each block in chunk-major order, a chunk being 16 bytes of one token:
  bf16:  element (c*16 + t)*8 + e  = X[t][8c + e]
  e4m3:  element (c*16 + t)*16 + e = X[t][16c + e]
"""

from __future__ import annotations

import numpy as np

PAGE = 16
LOCAL_D = 256
GLOBAL_D = 512
GLOBAL_ROT = 128


# ----------------------------------------------------------------------------
# byte model
# ----------------------------------------------------------------------------
def local_bytes_per_token(num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V for every KV head of one local layer."""
    return 2 * num_kv_heads * head_dim * elem_bytes


def global_bytes_per_token(head_dim: int, rot_dim: int, compressed: bool, elem_bytes: int = 2) -> int:
    """One global layer: full K+V, or V plus the rotated part of K."""
    return (head_dim + rot_dim) * elem_bytes if compressed else 2 * head_dim * elem_bytes


def local_page_bytes(num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return PAGE * local_bytes_per_token(num_kv_heads, head_dim, elem_bytes)


def global_page_bytes(head_dim: int, rot_dim: int, compressed: bool, elem_bytes: int = 2) -> int:
    return PAGE * global_bytes_per_token(head_dim, rot_dim, compressed, elem_bytes)


# ----------------------------------------------------------------------------
# element index maps inside one block
# ----------------------------------------------------------------------------
def local_k_index(elem_bytes: int) -> np.ndarray:
    """idx[t, d] = element offset of K[t][d] inside a local K block."""
    t = np.arange(PAGE)[:, None]
    d = np.arange(LOCAL_D)[None, :]
    c = d // 64
    if elem_bytes == 2:
        k, e = (d % 64) // 8, d % 8
        return ((k * 16 + t) * 4 + c) * 8 + e
    k, e = (d % 64) // 16, d % 16
    return ((k * 16 + t) * 4 + c) * 16 + e


def local_v_index(elem_bytes: int) -> np.ndarray:
    """idx[t, d] = element offset of V[t][d] inside a local V block."""
    t = np.arange(PAGE)[:, None]
    d = np.arange(LOCAL_D)[None, :]
    l, j = d // 4, d % 4
    if elem_bytes == 2:
        u, i = t // 2, t % 2
        return ((u * 64 + l) * 4 + j) * 2 + i
    u, i = t // 4, t % 4
    return ((u * 64 + l) * 4 + j) * 4 + i


def chunk_index(width: int, elem_bytes: int = 2) -> np.ndarray:
    """idx[t, d] = element offset of X[t][d] in a chunk-major [16][width]
    block whose chunks are 16 bytes (8 bf16 or 16 e4m3 elements) of a token."""
    e = 16 // elem_bytes
    t = np.arange(PAGE)[:, None]
    d = np.arange(width)[None, :]
    return ((d // e) * 16 + t) * e + d % e


# ----------------------------------------------------------------------------
# decoders: pool bytes -> contiguous codes of one sequence
# ----------------------------------------------------------------------------
def _pages_of(page_row, L):
    n = (L + PAGE - 1) // PAGE
    return np.asarray(page_row[:n], dtype=np.int64)


def local_codes(pool_bytes: np.ndarray, page_row, L: int, num_kv_heads: int,
                elem_bytes: int):
    """Contiguous K, V codes [L][Hkv][256] of one sequence from a local pool.

    pool_bytes: the whole pool as uint8.  Codes are uint16 (bf16) or uint8
    (e4m3).  Tokens in pages whose table entry is negative read as the
    all-ones code (0xFFFF / 0xFF), which is NaN in both formats.
    """
    dt = np.uint16 if elem_bytes == 2 else np.uint8
    block = PAGE * LOCAL_D
    elems = np.asarray(pool_bytes, dtype=np.uint8).view(dt)
    per_page = num_kv_heads * 2 * block
    ki = local_k_index(elem_bytes)
    vi = local_v_index(elem_bytes)
    pages = _pages_of(page_row, L)
    K = np.full((len(pages) * PAGE, num_kv_heads, LOCAL_D), np.iinfo(dt).max, dtype=dt)
    V = K.copy()
    for lp, pp in enumerate(pages):
        if pp < 0:
            continue
        base = pp * per_page
        for h in range(num_kv_heads):
            kb = elems[base + (2 * h) * block: base + (2 * h + 1) * block]
            vb = elems[base + (2 * h + 1) * block: base + (2 * h + 2) * block]
            K[lp * PAGE:(lp + 1) * PAGE, h, :] = kb[ki]
            V[lp * PAGE:(lp + 1) * PAGE, h, :] = vb[vi]
    return K[:L], V[:L]


def global_codes(pool_bytes: np.ndarray, page_row, L: int, compressed: bool, elem_bytes: int = 2):
    """Contiguous codes of one sequence from a global pool, uint16 (bf16)
    or uint8 (e4m3); unwritten pages read as the all-ones code (NaN).

    compressed: returns (V [L][512], K_rot [L][128]);
    full:       returns (K [L][512], V [L][512]).
    """
    dt = np.uint16 if elem_bytes == 2 else np.uint8
    elems = np.asarray(pool_bytes, dtype=np.uint8).view(dt)
    pages = _pages_of(page_row, L)
    if compressed:
        per_page = PAGE * (GLOBAL_D + GLOBAL_ROT)
        widths = (GLOBAL_D, GLOBAL_ROT)
    else:
        per_page = PAGE * 2 * GLOBAL_D
        widths = (GLOBAL_D, GLOBAL_D)
    A = np.full((len(pages) * PAGE, widths[0]), np.iinfo(dt).max, dtype=dt)
    B = np.full((len(pages) * PAGE, widths[1]), np.iinfo(dt).max, dtype=dt)
    ia, ib = chunk_index(widths[0], elem_bytes), chunk_index(widths[1], elem_bytes)
    for lp, pp in enumerate(pages):
        if pp < 0:
            continue
        base = pp * per_page
        a = elems[base: base + PAGE * widths[0]]
        b = elems[base + PAGE * widths[0]: base + per_page]
        A[lp * PAGE:(lp + 1) * PAGE] = a[ia]
        B[lp * PAGE:(lp + 1) * PAGE] = b[ib]
    return A[:L], B[:L]
