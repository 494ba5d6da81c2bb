"""Rotary position embedding in fp64.

Test infrastructure only (see ``oracle/__init__``).

pegainfer "Gemma 4" page, Architecture notes (table rows "Local RoPE" and
"Global RoPE", and the bullet on proportional RoPE):

* local layers rotate all 256 dims of the head with theta = 1e4;
* global layers rotate only 128 of the 512 dims with theta = 1e6, and the
  frequency denominator stays the full head dimension (512), so the rotated
  block uses the first 64 frequencies of a 512-dim rotary embedding.

Frequency of pair i: inv_freq_i = theta ** (-2 i / head_dim),
i = 0 .. rot_dim/2 - 1; angle = pos * inv_freq_i.

Pairing (the pages do not say): rotate-half inside the rotated block, pair
(i, i + rot_dim/2):
    y_i            = x_i cos - x_{i+R/2} sin
    y_{i+R/2}      = x_{i+R/2} cos + x_i sin
Dims at or past rot_dim pass through unchanged.
"""

from __future__ import annotations

import numpy as np

LOCAL_THETA = 1.0e4
GLOBAL_THETA = 1.0e6


def inv_freq(rot_dim: int, head_dim: int, theta: float) -> np.ndarray:
    """theta ** (-2 i / head_dim) for i in [0, rot_dim / 2), fp64."""
    i = np.arange(rot_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / np.float64(head_dim))


def rotate(x, pos, rot_dim: int, head_dim: int, theta: float) -> np.ndarray:
    """Apply RoPE to x[..., head_dim] at integer positions pos[...] (fp64).

    ``pos`` broadcasts against ``x.shape[:-1]``.
    """
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == head_dim and rot_dim % 2 == 0 and rot_dim <= head_dim
    half = rot_dim // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq(rot_dim, head_dim, theta)
    c = np.cos(ang)
    s = np.sin(ang)
    a = x[..., :half]
    b = x[..., half:rot_dim]
    y = x.copy()
    y[..., :half] = a * c - b * s
    y[..., half:rot_dim] = b * c + a * s
    return y


def rotate_local(k, pos):
    """Local family: full 256-dim rotation, theta 1e4."""
    return rotate(k, pos, rot_dim=256, head_dim=256, theta=LOCAL_THETA)


def rotate_global(k, pos):
    """Global family: first 128 of 512 dims, theta 1e6, denominator 512."""
    return rotate(k, pos, rot_dim=128, head_dim=512, theta=GLOBAL_THETA)
