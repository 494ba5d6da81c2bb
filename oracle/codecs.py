"""bf16 and OCP e4m3 (E4M3FN) codecs, fp64 in, exact fp64 out.

Test infrastructure only (see ``oracle/__init__``).

Both encoders round an fp64 value to the nearest point of the target grid,
ties to even, by exact fp64 arithmetic: the value is split by ``frexp`` into
an exponent and a fraction, the fraction is scaled by a power of two so the
grid spacing becomes 1, and ``rint`` (IEEE round-half-even, exact on fp64)
picks the grid point.  Nothing here calls a library float conversion.

e4m3 follows the pages' fp8 KV format: pegainfer PR #1012 (Description)
stores the sliding family's K/V "as e4m3 at scale 1.0", i.e. the stored code
is e4m3(x) and the value read back is decode(code).  The variant is the OCP
E4M3FN one native to gfx950: exponent bias 7, three mantissa bits,
subnormals m * 2**-9, largest finite 448, no infinities, NaN = S.1111.111.
Encoding saturates: anything whose magnitude rounds above 448 (including
+-inf) becomes +-448; NaN stays NaN.
"""

from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# bf16: 1 sign, 8 exponent (bias 127), 7 mantissa bits.
# ----------------------------------------------------------------------------
_BF16_MIN_NORMAL_EXP = -126      # smallest normal is 2**-126
_BF16_MANT_BITS = 7
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def _round_to_grid(mag: np.ndarray, mant_bits: int, min_normal_exp: int) -> np.ndarray:
    """Round non-negative finite fp64 magnitudes to a binary float grid.

    The grid has ``mant_bits`` explicit mantissa bits and subnormals below
    2**min_normal_exp (spacing 2**(min_normal_exp - mant_bits) there).  The
    result is the exact fp64 value of the nearest grid point, ties to even,
    with no upper clamp (the callers decide overflow).
    """
    mag = np.asarray(mag, dtype=np.float64)
    _, e = np.frexp(mag)                  # mag = f * 2**e, f in [0.5, 1)
    e = e.astype(np.int64) - 1            # mag = (2f) * 2**e, 2f in [1, 2)
    e = np.maximum(e, min_normal_exp)     # subnormal range shares the min spacing
    spacing_exp = e - mant_bits
    scaled = np.ldexp(mag, -spacing_exp)  # exact: power-of-two scaling
    q = np.rint(scaled)                   # ties to even
    return np.ldexp(q, spacing_exp)


def bf16_round(x) -> np.ndarray:
    """fp64 -> nearest bf16 value (as fp64), RNE; overflow -> +-inf; NaN kept."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    nan = np.isnan(x)
    fin = np.isfinite(x)
    mag = np.abs(np.where(fin, x, 0.0))
    r = _round_to_grid(mag, _BF16_MANT_BITS, _BF16_MIN_NORMAL_EXP)
    # IEEE RNE overflow: anything at or above the midpoint between the
    # largest finite value and 2**128 rounds to infinity.
    r = np.where(r > _BF16_MAX, np.inf, r)
    out[fin] = np.copysign(r, x)[fin]
    out[~fin] = x[~fin]
    out[nan] = np.nan
    return out


def bf16_encode(x) -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), RNE.  NaN -> 0x7FC0 | sign."""
    x = np.asarray(x, dtype=np.float64)
    r = bf16_round(x)
    # every bf16 value is exactly an fp32 value whose low 16 bits are zero
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        sign = (np.signbit(x[nan]).astype(np.uint16) << 15)
        bits[nan] = np.uint16(0x7FC0) | sign
    return bits


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):   # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# OCP e4m3 (E4M3FN): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0
_E4M3_BIAS = 7
_E4M3_MANT_BITS = 3
_E4M3_MIN_NORMAL_EXP = 1 - _E4M3_BIAS     # -6


def e4m3_round(x) -> np.ndarray:
    """fp64 -> nearest e4m3 value (as fp64), RNE, saturating to +-448, NaN kept."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    mag = np.abs(np.where(nan, 0.0, x))
    mag = np.minimum(mag, 2.0 * E4M3_MAX)  # inf and huge values saturate below
    r = _round_to_grid(mag, _E4M3_MANT_BITS, _E4M3_MIN_NORMAL_EXP)
    r = np.minimum(r, E4M3_MAX)
    out = np.copysign(r, np.where(nan, 1.0, x))
    out[nan] = np.nan
    return out


def e4m3_encode(x) -> np.ndarray:
    """fp64 -> e4m3 codes (uint8): RNE, saturating, NaN -> 0x7F | sign."""
    x = np.asarray(x, dtype=np.float64)
    r = e4m3_round(x)
    nan = np.isnan(r)
    mag = np.abs(np.where(nan, 0.0, r))
    sign = np.signbit(np.where(nan, x, r)).astype(np.uint8) << 7
    _, e = np.frexp(mag)
    e = e.astype(np.int64) - 1
    normal = mag >= 2.0 ** _E4M3_MIN_NORMAL_EXP
    # normal: mag = (1 + m/8) * 2**e, field = e + 7
    m_norm = np.rint(np.ldexp(mag, -e) * 8.0 - 8.0)
    # subnormal: mag = m * 2**-9
    m_sub = np.rint(np.ldexp(mag, 9))
    exp_field = np.where(normal, e + _E4M3_BIAS, 0)
    mant = np.where(normal, m_norm, m_sub)
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    code = np.where(nan, 0x7F, code).astype(np.uint8) | sign
    return code.astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """e4m3 codes (uint8) -> exact fp64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, ef - _E4M3_BIAS)
    sub = np.ldexp(m.astype(np.float64), -9)
    v = s * np.where(ef == 0, sub, normal)
    v = np.where((ef == 0xF) & (m == 0x7), np.nan, v)
    return v


def bf16_then_e4m3(x) -> np.ndarray:
    """The fp8 pool's store rounding: fp64 -> bf16 (RNE) -> e4m3 (RNE, sat).

    The local fp8 pool holds exactly e4m3(the bf16 pool's values): the K/V
    that would have been stored as bf16 are rounded once more to e4m3.
    Returns e4m3 codes.
    """
    return e4m3_encode(bf16_round(x))
