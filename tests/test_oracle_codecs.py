"""Pins for the oracle's bf16 and e4m3 codecs (CPU only).

Pinned against: the formats' definitions at hand-picked points (exact bit
patterns and ties), and the torch CPU casts (library routines) for
bf16 and for non-saturating e4m3.
"""

import numpy as np
import pytest
import torch

from oracle import codecs as C


# ---------------------------------------------------------------- bf16 ----
@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80),
    (-2.0, 0xC000),
    (0.5, 0x3F00),
    (1.0 + 2.0 ** -8, 0x3F80),            # exact tie -> even mantissa (0)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),        # exact tie -> even mantissa (2)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # just above the tie
    (2.0 ** -133, 0x0001),                # smallest subnormal
    (2.0 ** -134, 0x0000),                # tie between 0 and it -> 0
    (3 * 2.0 ** -134, 0x0002),            # tie between 1 and 2 -> 2
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),   # largest finite
    (3.5e38, 0x7F80),                     # overflow -> inf
    (float("inf"), 0x7F80),
    (-0.0, 0x8000),
])
def test_bf16_points(x, bits):
    assert int(C.bf16_encode(np.array([x]))[0]) == bits


def test_bf16_nan():
    b = C.bf16_encode(np.array([np.nan]))[0]
    assert (int(b) & 0x7F80) == 0x7F80 and (int(b) & 0x7F) != 0


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    # wide exponent spread, including subnormal fp32 and bf16 ranges
    x = (rng.standard_normal(400_000) * np.exp2(rng.integers(-140, 120, 400_000))).astype(np.float32)
    x = np.concatenate([x, rng.standard_normal(100_000).astype(np.float32)])
    ours = C.bf16_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_roundtrip_all_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = C.bf16_decode(b)
    fin = ~np.isnan(v)
    assert np.array_equal(C.bf16_encode(v[fin]), b[fin])
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ref), ~fin)
    assert np.array_equal(ref[fin], v[fin])


# ---------------------------------------------------------------- e4m3 ----
@pytest.mark.parametrize("code,val", [
    (0x00, 0.0), (0x80, -0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
    (0x08, 2.0 ** -6), (0x38, 1.0), (0x39, 1.125), (0x40, 2.0),
    (0x7E, 448.0), (0xFE, -448.0), (0x77, 240.0), (0x3F, 1.875),
])
def test_e4m3_decode_points(code, val):
    got = C.e4m3_decode(np.array([code], dtype=np.uint8))[0]
    assert got == val and np.signbit(got) == np.signbit(val)


def test_e4m3_nan_codes():
    d = C.e4m3_decode(np.arange(256, dtype=np.uint32).astype(np.uint8))
    assert np.isnan(d).sum() == 2 and np.isnan(d[0x7F]) and np.isnan(d[0xFF])


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    ours = C.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_e4m3_roundtrip_finite_codes():
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    v = C.e4m3_decode(codes)
    fin = ~np.isnan(v)
    assert np.array_equal(C.e4m3_encode(v[fin]), codes[fin])


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),            # tie between 1 and 1.125 -> even (1.0)
    (1.1875, 0x3A),            # tie between 1.125 and 1.25 -> even (1.25)
    (2.0 ** -10, 0x00),        # tie between 0 and the smallest subnormal -> 0
    (3 * 2.0 ** -10, 0x02),    # tie between 1 and 2 subnormal steps -> 2
    (464.0, 0x7E),             # would round to 480 -> saturates to 448
    (449.0, 0x7E),
    (1e6, 0x7E), (float("inf"), 0x7E), (-float("inf"), 0xFE), (-500.0, 0xFE),
])
def test_e4m3_encode_points(x, code):
    assert int(C.e4m3_encode(np.array([x]))[0]) == code


def test_e4m3_encode_nan():
    assert int(C.e4m3_encode(np.array([np.nan]))[0]) & 0x7F == 0x7F


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(300_000) * np.exp2(rng.integers(-12, 9, 300_000))).astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    ours = C.e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_store_is_double_rounded():
    # 1 + 1/16 + 2**-12 rounds to 1.0625 in bf16, a tie for e4m3 that goes to
    # 1.0; rounding the fp64 value straight to e4m3 would give 1.125.
    x = np.array([1.0 + 1.0 / 16 + 2.0 ** -12])
    assert int(C.bf16_then_e4m3(x)[0]) == 0x38
    assert int(C.e4m3_encode(x)[0]) == 0x39
