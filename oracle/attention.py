"""Naive masked softmax attention over contiguous K/V, fp64.

Test infrastructure only (see ``oracle/__init__``).

What the hot path computes, from the pages:

* pegainfer "Gemma 4" page, intro and Architecture notes: local layers attend
  with a sliding window of 1024 tokens at head dim 256, grouped-query (16 q
  heads over 8 KV heads on the 12B line); global layers attend over the whole
  context at head dim 512 with a single KV head.
* pegainfer "Gemma 4" page, Scheduling: every active request advances one
  token per step; a new prompt's rows are computed in the same step.

Readings where the pages are silent (each listed in the design notes):

* a query at position p attends the keys at positions j with
  lo <= j <= p, lo = max(0, p - W + 1) for the local family and 0 for the
  global family -- i.e. exactly min(p + 1, W) keys, itself included;
* the current token's K/V is in the cache when it attends, so a sequence of
  L tokens whose last q_len tokens are queries has its query rows at
  positions L - q_len .. L - 1;
* q head h reads KV head floor(h / G), G = Hq / Hkv;
* the softmax scale is a parameter (1/sqrt(head_dim) in every workload);
* no logit soft-capping inside attention (the pages cap only final logits).

Each output is
    z_j = scale * sum_d q[h, d] * K[j, g, d]    for j in the window, -inf else
    w   = exp(z - max z) / sum exp(z - max z)
    out = sum_j w_j V[j, g, :]
materialised in full, in fp64.
"""

from __future__ import annotations

import math

import numpy as np

from . import rope as _rope


def window_lo(p: int, window: int | None) -> int:
    """First attended key position for a query at position p."""
    if window is None:
        return 0
    return max(0, p - window + 1)


def attend(q, K, V, q_pos, scale: float, window: int | None = None,
           return_weights: bool = False, max_elems: int = 1 << 25):
    """Attention of query rows over one sequence's contiguous keys.

    q      : [R, Hq, D]   fp64 (already rotated)
    K, V   : [L, Hkv, D]  fp64 (K already rotated)
    q_pos  : [R] int, positions of the query rows (each < L)
    window : sliding window W (local family) or None (global family)

    Returns out [R, Hq, D] fp64 (and weights [R, Hq, L] if asked).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    R, Hq, D = q.shape
    L, Hkv, Dk = K.shape
    assert Dk == D and V.shape == K.shape and q_pos.shape == (R,)
    assert Hq % Hkv == 0
    G = Hq // Hkv
    assert (q_pos < L).all() and (q_pos >= 0).all()

    out = np.empty((R, Hq, D), dtype=np.float64)
    weights = np.zeros((R, Hq, L), dtype=np.float64) if return_weights else None
    lo_all = np.array([window_lo(int(p), window) for p in q_pos], dtype=np.int64)
    # Only keys inside a row's own range [lo, p] enter its sum; keys outside
    # are never read, so unwritten (NaN) slots elsewhere cannot leak in.
    # Rows go in blocks over the union of their ranges; a block whose union
    # holds a non-finite key or value falls back to one row at a time.
    rows_per_block = max(1, max_elems // max(1, Hq * L))
    for r0 in range(0, R, rows_per_block):
        r1 = min(R, r0 + rows_per_block)
        ja, jb = int(lo_all[r0:r1].min()), int(q_pos[r0:r1].max()) + 1
        if np.isfinite(K[ja:jb]).all() and np.isfinite(V[ja:jb]).all():
            _attend_block(q, K, V, q_pos, lo_all, scale, G, r0, r1, ja, jb, out, weights)
        else:
            for r in range(r0, r1):
                _attend_block(q, K, V, q_pos, lo_all, scale, G, r, r + 1,
                              int(lo_all[r]), int(q_pos[r]) + 1, out, weights)
    if return_weights:
        return out, weights
    return out


def _attend_block(q, K, V, q_pos, lo_all, scale, G, r0, r1, ja, jb, out, weights):
    """Rows r0..r1-1 over keys ja..jb-1 (the union of their ranges)."""
    Hkv = K.shape[1]
    j = np.arange(ja, jb)
    allowed = (j[None, :] >= lo_all[r0:r1, None]) & (j[None, :] <= q_pos[r0:r1, None])  # [r, n]
    for g in range(Hkv):
        qg = q[r0:r1, g * G:(g + 1) * G, :]               # [r, G, D]
        z = scale * (qg @ K[ja:jb, g, :].T)               # [r, G, n]
        z = np.where(allowed[:, None, :], z, -np.inf)
        zmax = z.max(axis=-1, keepdims=True)
        e = np.exp(z - zmax)                              # exactly 0 where masked
        w = e / e.sum(axis=-1, keepdims=True)
        out[r0:r1, g * G:(g + 1) * G, :] = w @ V[ja:jb, g, :]
        if weights is not None:
            weights[r0:r1, g * G:(g + 1) * G, ja:jb] = w


def attend_scalar(q, K, V, q_pos, scale: float, window: int | None = None):
    """The same definition as ``attend`` in plain Python loops (tiny inputs).

    Uses math.exp and math.fsum (exactly rounded sums), one output element at a
    time; an independent formulation for pinning ``attend``.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    R, Hq, D = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.zeros((R, Hq, D), dtype=np.float64)
    for r in range(R):
        p = int(q_pos[r])
        lo = window_lo(p, window)
        for h in range(Hq):
            g = h // G
            keys = range(lo, p + 1)
            z = [scale * math.fsum(float(q[r, h, d]) * float(K[jj, g, d]) for d in range(D))
                 for jj in keys]
            zm = max(z)
            e = [math.exp(zz - zm) for zz in z]
            s = math.fsum(e)
            for d in range(D):
                out[r, h, d] = math.fsum(e[i] * float(V[jj, g, d]) for i, jj in enumerate(keys)) / s
    return out


def attend_sequence(q_rows, K, V, scale: float, window: int | None = None, **kw):
    """Query rows are the last q_len tokens of a sequence of L = K.shape[0].

    Row r sits at position L - q_len + r (its own K/V is already in K, V).
    """
    q_rows = np.asarray(q_rows)
    L = K.shape[0]
    q_len = q_rows.shape[0]
    pos = np.arange(L - q_len, L)
    return attend(q_rows, K, V, pos, scale, window, **kw)


def k_from_compressed(v, k_rot):
    """Rebuild a global-layer K from its compressed record.

    Gewell post, "the Why": K and V are tied on global layers and RoPE rotates
    only 25% of K, so storing V and the rotated quarter of K is enough:
    K = [K_rot (dims 0..127) | V[128:512]].
    """
    v = np.asarray(v, dtype=np.float64)
    k_rot = np.asarray(k_rot, dtype=np.float64)
    r = k_rot.shape[-1]
    return np.concatenate([k_rot, v[..., r:]], axis=-1)


def global_k(v, pos, w_k=None):
    """A global layer's K at positions pos, from its V and K's norm weight.

    pegainfer "Gemma 4" page, Architecture notes: V is the K projection's
    output after a norm with no scale; K is that same output after k_norm,
    whose learned per-dim weight w_k is the only difference, and then the
    proportional RoPE (first 128 of 512 dims).  So K = RoPE(V * w_k); with
    w_k None (or all ones) K is V before rotation, the tied store.
    """
    v = np.asarray(v, dtype=np.float64)
    k = v if w_k is None else v * np.asarray(w_k, dtype=np.float64)
    return _rope.rotate_global(k, pos)
