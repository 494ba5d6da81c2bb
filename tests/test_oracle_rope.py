"""Pins for the oracle's rotary embedding (CPU only).

Pinned against: the identity at position 0, rotation invariants (pair norms,
relative-position property), a complex-number formulation built on numpy's
complex exponential and ``logspace`` (a different route to the same
frequencies), and the pages' statement that the proportional global RoPE
keeps the full 512-dim frequency denominator (pegainfer "Gemma 4" page,
Architecture notes).
"""

import numpy as np
import pytest

from oracle import rope as R


@pytest.mark.parametrize("rot,dim,theta", [(256, 256, 1e4), (128, 512, 1e6)])
def test_pos0_identity(rot, dim, theta):
    x = np.random.default_rng(0).standard_normal((5, dim))
    assert np.array_equal(R.rotate(x, np.zeros(5), rot, dim, theta), x)


@pytest.mark.parametrize("rot,dim,theta", [(256, 256, 1e4), (128, 512, 1e6)])
def test_pair_norms_and_passthrough(rot, dim, theta):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, dim))
    pos = rng.integers(0, 200_000, 7)
    y = R.rotate(x, pos, rot, dim, theta)
    h = rot // 2
    nx = x[:, :h] ** 2 + x[:, h:rot] ** 2
    ny = y[:, :h] ** 2 + y[:, h:rot] ** 2
    assert np.max(np.abs(nx - ny)) < 1e-12 * max(1.0, nx.max())
    assert np.array_equal(y[:, rot:], x[:, rot:])


@pytest.mark.parametrize("rot,dim,theta", [(256, 256, 1e4), (128, 512, 1e6)])
def test_relative_position(rot, dim, theta):
    rng = np.random.default_rng(2)
    a = rng.standard_normal(dim)
    b = rng.standard_normal(dim)
    a[rot:] = 0
    b[rot:] = 0
    for m, n in [(10, 3), (5000, 4990), (131071, 7)]:
        lhs = R.rotate(a, m, rot, dim, theta) @ R.rotate(b, n, rot, dim, theta)
        rhs = R.rotate(a, m - n, rot, dim, theta) @ b
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(lhs))


def test_first_pair_turns_by_pos_radians():
    # pair 0 has frequency 1: e_0 at position p goes to (cos p, sin p) in the
    # (0, R/2) plane -- pins pairing and direction of rotation
    for rot, dim, theta in [(256, 256, 1e4), (128, 512, 1e6)]:
        x = np.zeros(dim)
        x[0] = 1.0
        y = R.rotate(x, 3, rot, dim, theta)
        assert np.isclose(y[0], np.cos(3.0), atol=1e-15)
        assert np.isclose(y[rot // 2], np.sin(3.0), atol=1e-15)
        assert np.count_nonzero(y) == 2


@pytest.mark.parametrize("rot,dim,theta", [(256, 256, 1e4), (128, 512, 1e6)])
def test_matches_complex_formulation(rot, dim, theta):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((9, dim))
    pos = rng.integers(0, 262_144, 9)
    h = rot // 2
    # frequencies theta^(-2i/dim), i < h, as a log-spaced sequence
    f = np.logspace(0.0, -(rot - 2) / dim * np.log10(theta), h)
    z = (x[:, :h] + 1j * x[:, h:rot]) * np.exp(1j * pos[:, None] * f[None, :])
    y = R.rotate(x, pos, rot, dim, theta)
    assert np.max(np.abs(y[:, :h] - z.real)) < 1e-9
    assert np.max(np.abs(y[:, h:rot] - z.imag)) < 1e-9


def test_proportional_rope_keeps_full_denominator():
    # The global rotation of dims [0,128) uses the first 64 frequencies of a
    # full 512-dim rotation: put the same pair at (i, i+64) and at (i, i+256).
    rng = np.random.default_rng(4)
    for i in [0, 1, 17, 63]:
        a, b = rng.standard_normal(2)
        xp = np.zeros(512)
        xp[i], xp[i + 64] = a, b
        xf = np.zeros(512)
        xf[i], xf[i + 256] = a, b
        for pos in [1, 777, 131071]:
            yp = R.rotate_global(xp, pos)
            yf = R.rotate(xf, pos, 512, 512, R.GLOBAL_THETA)
            assert np.isclose(yp[i], yf[i], rtol=0, atol=1e-12)
            assert np.isclose(yp[i + 64], yf[i + 256], rtol=0, atol=1e-12)
