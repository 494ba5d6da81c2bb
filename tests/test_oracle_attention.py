"""Pins for the oracle's masked softmax attention (CPU only).

Pinned against: an independent scalar formulation (math.fsum / math.exp),
closed forms (single key, window of one, zero query, constant V, a dominant
key), invariants (weights sum to one, exact zeros outside the window, equal
heads give equal outputs, a wide window equals global causal attention), the
compressed global record's K rebuild, and torch's CPU
``scaled_dot_product_attention`` in fp64 with an explicit mask (a library
routine).
"""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import rope as R


def _rand(rng, L, Hkv, D, R_, Hq):
    q = rng.standard_normal((R_, Hq, D))
    K = rng.standard_normal((L, Hkv, D))
    V = rng.standard_normal((L, Hkv, D))
    return q, K, V


@pytest.mark.parametrize("L,W,Hq,Hkv,D", [(1, 4, 2, 1, 3), (7, 3, 2, 1, 5), (13, 5, 4, 2, 4),
                                          (20, None, 3, 1, 6), (16, 16, 2, 2, 8), (9, 1, 2, 1, 2)])
def test_matches_scalar_formulation(L, W, Hq, Hkv, D):
    rng = np.random.default_rng(L * 100 + D)
    q, K, V = _rand(rng, L, Hkv, D, 4, Hq)
    pos = rng.integers(0, L, 4)
    a = A.attend(q, K, V, pos, 0.37, W)
    b = A.attend_scalar(q, K, V, pos, 0.37, W)
    assert np.max(np.abs(a - b)) < 1e-12


def test_single_key():
    rng = np.random.default_rng(0)
    q, K, V = _rand(rng, 1, 1, 8, 1, 2)
    out = A.attend(q, K, V, [0], 1.0, 4)
    assert np.allclose(out, V[0, 0][None, None, :], atol=0, rtol=1e-15)


def test_window_of_one_returns_own_value():
    rng = np.random.default_rng(1)
    q, K, V = _rand(rng, 30, 2, 8, 5, 4)
    pos = np.array([0, 3, 17, 28, 29])
    out = A.attend(q, K, V, pos, 0.5, 1)
    for r, p in enumerate(pos):
        for h in range(4):
            assert np.array_equal(out[r, h], V[p, h // 2])


def test_zero_query_is_window_mean():
    rng = np.random.default_rng(2)
    _, K, V = _rand(rng, 50, 1, 6, 1, 1)
    q = np.zeros((3, 2, 6))
    pos = np.array([5, 30, 49])
    out = A.attend(q, K, V, pos, 1.0, 8)
    for r, p in enumerate(pos):
        lo = max(0, p - 7)
        assert np.allclose(out[r, 0], V[lo:p + 1, 0].mean(axis=0), atol=1e-14)


def test_constant_values():
    rng = np.random.default_rng(3)
    q, K, _ = _rand(rng, 40, 2, 8, 3, 4)
    V = np.broadcast_to(rng.standard_normal((1, 2, 8)), (40, 2, 8))
    out = A.attend(q, K, V, [10, 20, 39], 0.3, 16)
    for h in range(4):
        assert np.allclose(out[:, h], V[0, h // 2][None], atol=1e-14)


def test_dominant_key():
    rng = np.random.default_rng(4)
    q, K, V = _rand(rng, 64, 1, 16, 1, 2)
    for j in [32, 40, 63]:
        Kd = K.copy()
        Kd[j, 0] = 300.0 * q[0, 0] / np.linalg.norm(q[0, 0])
        out = A.attend(q[:, :1], Kd, V, [63], 1.0, 32)
        assert np.allclose(out[0, 0], V[j, 0], atol=1e-12)


def test_weights_sum_to_one_and_vanish_outside_window():
    rng = np.random.default_rng(5)
    q, K, V = _rand(rng, 100, 2, 8, 6, 4)
    pos = np.array([0, 1, 31, 32, 70, 99])
    W = 32
    _, w = A.attend(q, K, V, pos, 0.5, W, return_weights=True)
    assert np.max(np.abs(w.sum(-1) - 1.0)) < 1e-12
    for r, p in enumerate(pos):
        lo = max(0, p - W + 1)
        assert np.all(w[r, :, :lo] == 0.0) and np.all(w[r, :, p + 1:] == 0.0)
        assert np.all(w[r, :, lo:p + 1] > 0.0)
        assert (p + 1 - lo) == min(p + 1, W)


def test_equal_heads_in_group_agree():
    rng = np.random.default_rng(6)
    q, K, V = _rand(rng, 33, 2, 8, 2, 4)
    q[:, 1] = q[:, 0]
    out = A.attend(q, K, V, [20, 32], 0.4, 16)
    assert np.array_equal(out[:, 0], out[:, 1])


def test_wide_window_is_global_causal():
    rng = np.random.default_rng(7)
    q, K, V = _rand(rng, 25, 1, 8, 4, 2)
    pos = np.array([0, 5, 12, 24])
    assert np.array_equal(A.attend(q, K, V, pos, 0.5, 25), A.attend(q, K, V, pos, 0.5, None))
    assert np.array_equal(A.attend(q, K, V, pos, 0.5, 10_000), A.attend(q, K, V, pos, 0.5, None))


def test_attend_sequence_positions():
    rng = np.random.default_rng(8)
    q, K, V = _rand(rng, 12, 1, 4, 3, 1)
    a = A.attend_sequence(q, K, V, 0.5, 4)
    b = A.attend(q, K, V, [9, 10, 11], 0.5, 4)
    assert np.array_equal(a, b)


def test_compressed_record_rebuilds_full_k():
    rng = np.random.default_rng(9)
    L = 40
    v = rng.standard_normal((L, 512))
    k_full = R.rotate_global(v, np.arange(L))      # K = V before rotation (tied)
    k_rot = k_full[:, :128]
    k = A.k_from_compressed(v, k_rot)
    assert np.array_equal(k, k_full)
    q = rng.standard_normal((1, 32, 512))
    o1 = A.attend(q, k[:, None], v[:, None], [L - 1], 512 ** -0.5, None)
    o2 = A.attend(q, k_full[:, None], v[:, None], [L - 1], 512 ** -0.5, None)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("L,W,Hq,Hkv,D", [(300, 64, 4, 2, 32), (257, None, 8, 1, 64), (128, 1, 2, 1, 16)])
def test_matches_torch_sdpa(L, W, Hq, Hkv, D):
    rng = np.random.default_rng(L)
    q, K, V = _rand(rng, L, Hkv, D, 5, Hq)
    pos = np.sort(rng.integers(0, L, 5))
    pos[-1] = L - 1
    scale = 1.0 / np.sqrt(D)
    ours = A.attend(q, K, V, pos, scale, W)
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                                  # [Hq, R, D]
    Kt = torch.from_numpy(np.repeat(K, G, axis=1)).permute(1, 0, 2).contiguous()
    Vt = torch.from_numpy(np.repeat(V, G, axis=1)).permute(1, 0, 2).contiguous()
    j = torch.arange(L)
    p = torch.from_numpy(pos)
    lo = torch.zeros_like(p) if W is None else torch.clamp(p - W + 1, min=0)
    mask = (j[None, :] <= p[:, None]) & (j[None, :] >= lo[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask, scale=scale)
    ref = ref.permute(1, 0, 2).numpy()
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_keys_outside_the_window_are_never_read():
    # NaN in K/V outside every row's [lo, p] must not reach any output
    rng = np.random.default_rng(10)
    q, K, V = _rand(rng, 90, 2, 8, 3, 4)
    pos = np.array([40, 55, 60])
    ref = A.attend(q, K, V, pos, 0.5, 16)
    Kn, Vn = K.copy(), V.copy()
    Kn[:25], Vn[:25] = np.nan, np.nan       # before the first row's window
    Kn[61:], Vn[61:] = np.inf, np.nan       # after the last row
    Kn[30:40, 1], Vn[30:40, 1] = np.nan, np.nan   # inside the union, outside row 1/2 windows
    got = A.attend(q[1:], Kn, Vn, pos[1:], 0.5, 16)
    assert np.isfinite(got).all() and np.max(np.abs(got - ref[1:])) < 1e-13
    got0 = A.attend(q[:1], Kn, Vn, pos[:1], 0.5, 16)   # row 0's window 25..40 holds NaN at 30..39
    assert np.isnan(got0[0, 2:]).all()      # heads of KV head 1 read it: NaN propagates
    assert np.max(np.abs(got0[0, :2] - ref[0, :2])) < 1e-13


def test_global_k_with_unit_weight_is_the_tied_k():
    rng = np.random.default_rng(21)
    v = rng.standard_normal((30, 512))
    pos = rng.integers(0, 100000, size=30)
    assert np.array_equal(A.global_k(v, pos), R.rotate_global(v, pos))
    assert np.array_equal(A.global_k(v, pos, np.ones(512)), R.rotate_global(v, pos))


def test_global_k_weight_applies_before_rotation():
    """Dims 128..511 never rotate, so there K is V * w_k itself; dims 0..127
    are a rotation of (V * w_k) in the pairs (i, i + 64), which keeps each
    pair's length.  Weighting after rotation would break the second."""
    rng = np.random.default_rng(22)
    v = rng.standard_normal((25, 512))
    w = rng.uniform(0.25, 2.0, size=512)
    pos = rng.integers(1, 200000, size=25)
    k = A.global_k(v, pos, w)
    kw = v * w
    assert np.array_equal(k[:, 128:], kw[:, 128:])
    np.testing.assert_allclose(k[:, :64] ** 2 + k[:, 64:128] ** 2,
                               kw[:, :64] ** 2 + kw[:, 64:128] ** 2, rtol=1e-12)
    assert not np.allclose(k[:, :128], kw[:, :128])
    after = R.rotate_global(v, pos)[:, :128] * w[:128]
    assert not np.allclose(after[:, :64] ** 2 + after[:, 64:128] ** 2,
                           kw[:, :64] ** 2 + kw[:, 64:128] ** 2)


def test_norm_weight_folds_into_q():
    """Attention over K = RoPE(V * w_k) equals attention over the stored record
    (rotated quarter of that K, V for dims 128..511) with q's dims 128..511
    multiplied by w_k: each score sum_d q_d K_d is the same sum."""
    rng = np.random.default_rng(23)
    L = 50
    v = rng.standard_normal((L, 512))
    w = rng.uniform(0.25, 2.0, size=512)
    pos = np.arange(L)
    k = A.global_k(v, pos, w)
    q = rng.standard_normal((2, 8, 512))
    o_true = A.attend(q, k[:, None], v[:, None], [L - 2, L - 1], 512 ** -0.5, None)
    q_fold = q.copy()
    q_fold[..., 128:] *= w[128:]
    k_rec = A.k_from_compressed(v, k[:, :128])
    o_fold = A.attend(q_fold, k_rec[:, None], v[:, None], [L - 2, L - 1], 512 ** -0.5, None)
    np.testing.assert_allclose(o_fold, o_true, rtol=1e-12, atol=1e-13)
    # without the fold the weight is lost beyond dim 128
    o_nofold = A.attend(q, k_rec[:, None], v[:, None], [L - 2, L - 1], 512 ** -0.5, None)
    assert np.abs(o_nofold - o_true).max() > 1e-3
