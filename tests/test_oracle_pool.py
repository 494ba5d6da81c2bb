"""Pins for the oracle's byte model, pool layouts and layer pattern (CPU only).

Pinned against the numbers the pages print (tests/golden/pages_numbers.json,
each with its page and section) and against bijectivity of the documented
in-page layouts.
"""

import json
import os

import numpy as np
import pytest

from oracle import layers, pool

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
ARCH = GOLD["arch_12b"]


def test_compressed_global_ratio():
    full = pool.global_bytes_per_token(ARCH["global_head_dim"], ARCH["global_rope_dims"], False)
    comp = pool.global_bytes_per_token(ARCH["global_head_dim"], ARCH["global_rope_dims"], True)
    assert comp / full == GOLD["global_compressed_ratio"]["value"]
    assert ARCH["global_rope_dims"] / ARCH["global_head_dim"] == GOLD["rotated_fraction_of_global_k"]["value"]


def test_request_pool_bytes_12b():
    # one 8192-token request at the 12B geometry, every token of every layer
    # stored as bf16 with the full K/V global record: about 2.6 GiB
    loc = pool.local_bytes_per_token(ARCH["local_kv_heads"], ARCH["local_head_dim"], 2)
    glb = pool.global_bytes_per_token(ARCH["global_head_dim"], ARCH["global_rope_dims"], False)
    total = 8192 * (ARCH["local_layers"] * loc + ARCH["global_layers"] * glb)
    gib = total / 2 ** 30
    assert gib == pytest.approx(GOLD["request_pool_gib_at_8192_tokens"]["value"], abs=0.05)


def test_page_bytes():
    P = GOLD["page_size_tokens"]["value"]
    assert pool.PAGE == P
    assert pool.local_page_bytes(8, 256, 2) == P * 8 * 2 * 256 * 2 == 131072
    assert pool.local_page_bytes(8, 256, 1) == 65536
    assert pool.global_page_bytes(512, 128, True) == 20480
    assert pool.global_page_bytes(512, 128, False) == 32768
    assert pool.global_page_bytes(512, 128, True, 1) == 10240
    assert pool.global_page_bytes(512, 128, False, 1) == 16384
    # the e4m3 compressed record keeps the pages' 0.625x of the full one
    assert pool.global_page_bytes(512, 128, True, 1) / pool.global_page_bytes(512, 128, False, 1) == \
        GOLD["global_compressed_ratio"]["value"]


def test_layer_pattern_12b():
    g = layers.global_layers(ARCH["layers"])
    assert len(g) == ARCH["global_layers"]
    assert ARCH["layers"] - len(g) == ARCH["local_layers"]
    assert g[-1] == ARCH["layers"] - 1
    # five local layers before each global one
    assert all(not layers.is_global(i, 48) for i in range(5))


def test_layer_pattern_60():
    assert layers.global_layers(60) == [5, 11, 17, 23, 29, 35, 41, 47, 53, 59]


@pytest.mark.parametrize("eb", [1, 2])
def test_local_layouts_are_bijections(eb):
    for idx in (pool.local_k_index(eb), pool.local_v_index(eb)):
        assert idx.shape == (16, 256)
        assert np.array_equal(np.sort(idx.ravel()), np.arange(16 * 256))


@pytest.mark.parametrize("eb", [1, 2])
def test_chunk_layout_is_bijection(eb):
    for w in (128, 512):
        idx = pool.chunk_index(w, eb)
        assert np.array_equal(np.sort(idx.ravel()), np.arange(16 * w))
        # a chunk is 16 bytes of one token: consecutive dims, one token
        e = 16 // eb
        assert np.array_equal(idx[5, :e], idx[5, 0] + np.arange(e))
        assert idx[5, e] == idx[5, 0] + 16 * e


@pytest.mark.parametrize("eb", [1, 2])
@pytest.mark.parametrize("compressed", [True, False])
def test_global_decoder_roundtrip(eb, compressed):
    """Pages written element by element from the layout's formula read back
    in token order, through a shuffled page table."""
    rng = np.random.default_rng(10 + eb)
    dt = np.uint16 if eb == 2 else np.uint8
    e = 16 // eb
    wa, wb = (512, 128) if compressed else (512, 512)
    L, npages = 37, 6
    A = rng.integers(0, 2 ** (8 * eb) - 1, (48, wa)).astype(dt)
    B = rng.integers(0, 2 ** (8 * eb) - 1, (48, wb)).astype(dt)
    table = np.array([4, 1, 5], dtype=np.int32)
    per_page = 16 * (wa + wb)
    elems = np.zeros(npages * per_page, dtype=dt)
    for lp, pp in enumerate(table):
        for t in range(16):
            for d in range(wa):
                elems[pp * per_page + ((d // e) * 16 + t) * e + d % e] = A[lp * 16 + t, d]
            for d in range(wb):
                elems[pp * per_page + 16 * wa + ((d // e) * 16 + t) * e + d % e] = B[lp * 16 + t, d]
    Ad, Bd = pool.global_codes(elems.view(np.uint8), table, L, compressed, eb)
    assert np.array_equal(Ad, A[:L]) and np.array_equal(Bd, B[:L])


@pytest.mark.parametrize("eb", [1, 2])
def test_local_decoder_roundtrip(eb):
    rng = np.random.default_rng(eb)
    dt = np.uint16 if eb == 2 else np.uint8
    Hkv, L, npages = 2, 40, 5
    K = rng.integers(0, 2 ** (8 * eb) - 1, (48, Hkv, 256)).astype(dt)
    V = rng.integers(0, 2 ** (8 * eb) - 1, (48, Hkv, 256)).astype(dt)
    table = np.array([3, 0, 4], dtype=np.int32)     # logical page -> physical page
    per_page = Hkv * 2 * 16 * 256
    elems = np.zeros(npages * per_page, dtype=dt)
    ki, vi = pool.local_k_index(eb), pool.local_v_index(eb)
    for lp, pp in enumerate(table):
        for h in range(Hkv):
            kb = np.zeros(16 * 256, dtype=dt)
            vb = np.zeros(16 * 256, dtype=dt)
            kb[ki] = K[lp * 16:(lp + 1) * 16, h]
            vb[vi] = V[lp * 16:(lp + 1) * 16, h]
            base = pp * per_page + 2 * h * 4096
            elems[base:base + 4096] = kb
            elems[base + 4096:base + 8192] = vb
    Kd, Vd = pool.local_codes(elems.view(np.uint8), table, L, Hkv, eb)
    assert np.array_equal(Kd, K[:L]) and np.array_equal(Vd, V[:L])
