"""Oracle-side inputs for parity tests: the synthetic draws turned into the
contiguous fp64 K/V/q the CPU oracle attends over, using only ``oracle``
arithmetic (its own codecs and rotary embedding)."""

from __future__ import annotations

import numpy as np

from oracle import attention as OA
from oracle import codecs as OC
from oracle import rope as OR

# tolerances stated for the path: bf16 and e4m3 alike
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def local_seq(case, s):
    """fp64 K, V [L][Hkv][256] of sequence s as the pool holds them
    (NaN where no token was written)."""
    L = int(case.seqs.lens[s])
    sel = case.tok_seq == s
    pos = case.tok_pos[sel]
    Hkv = case.num_kv_heads
    K = np.full((L, Hkv, 256), np.nan)
    V = np.full((L, Hkv, 256), np.nan)
    k = OC.bf16_round(case.k[sel].astype(np.float64))
    v = OC.bf16_round(case.v[sel].astype(np.float64))
    if case.rope:
        k = OC.bf16_round(OR.rotate_local(k, pos[:, None]))
    if case.fp8:
        k = OC.e4m3_decode(OC.e4m3_encode(k))
        v = OC.e4m3_decode(OC.e4m3_encode(v))
    K[pos] = k
    V[pos] = v
    return K, V


def global_seq(case, s):
    """fp64 K, V [L][1][512] of global sequence s (K rebuilt from the record).

    With a norm weight on K (case.w_k), K before rotation is the model's
    bf16(V * w_k): its rotated quarter is stored rounded to bf16, and dims
    128..511 are that K itself, not V."""
    sel = case.tok_seq == s
    pos = case.tok_pos[sel]
    v = OC.bf16_round(case.v[sel].astype(np.float64))
    if case.w_k is None:
        k_rot = v[:, :128]
        if case.rope:
            k_rot = OC.bf16_round(OR.rotate_global(v, pos)[:, :128])
        k = OA.k_from_compressed(v, k_rot)
    else:
        k_pre = OC.bf16_round(v * case.w_k.astype(np.float64))
        k = OA.global_k(k_pre, pos if case.rope else np.zeros_like(pos))
        k[:, :128] = OC.bf16_round(k[:, :128])
    if case.fp8:
        # e4m3 pool: every stored element is the e4m3 code of its bf16 value
        k = OC.e4m3_decode(OC.e4m3_encode(k))
        v = OC.e4m3_decode(OC.e4m3_encode(v))
    L = int(case.seqs.lens[s])
    K = np.full((L, 512), np.nan)
    V = np.full((L, 512), np.nan)
    K[pos] = k
    V[pos] = v
    return K[:, None, :], V[:, None, :]


def q_rows(case, s):
    qi = case.q_indptr
    return OC.bf16_round(case.q[qi[s]:qi[s + 1]].astype(np.float64))


def oracle_out(case, seqs=None):
    """Oracle output rows of the chosen sequences: {s: [q_len, Hq, D]}."""
    local = hasattr(case, "window")
    res = {}
    for s in (range(case.seqs.S) if seqs is None else seqs):
        K, V = local_seq(case, s) if local else global_seq(case, s)
        res[s] = OA.attend_sequence(q_rows(case, s), K, V, case.scale,
                                    case.window if local else None)
    return res


def compare(gpu_rows: np.ndarray, ref_rows: np.ndarray, label: str = ""):
    """Assert the stated tolerances; return (max_abs, mean_abs, max_rel_rms)."""
    g = np.asarray(gpu_rows, dtype=np.float64)
    r = np.asarray(ref_rows, dtype=np.float64)
    assert g.shape == r.shape, (label, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{label}: non-finite GPU output"
    err = np.abs(g - r)
    mx, mean = float(err.max()), float(err.mean())
    rms = float(np.sqrt(np.mean(r * r))) or 1.0
    assert mx <= MAX_ABS, f"{label}: max abs err {mx:.3e} > {MAX_ABS}"
    assert mean <= MEAN_ABS, f"{label}: mean abs err {mean:.3e} > {MEAN_ABS}"
    return mx, mean, mx / rms
