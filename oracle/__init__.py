"""CPU fp64 oracle for paged hybrid-KV decode attention (Gemma 4 hybrid stack).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (``paged_hybrid_kv_amd``) and imports nothing from it; the two
meet only in the seeded input generators (``paged_hybrid_kv_amd.synth``),
which draw random numbers and do none of the method's arithmetic.

What it computes, from the pages it follows:

* ``codecs``    -- bf16 and OCP e4m3 (E4M3FN) rounding onto their grids, and
                   decoding back to fp64 (pegainfer PR #1012, Description:
                   e4m3 at scale 1.0 for the local family).
* ``rope``      -- rotary position embedding, full (local family: 256 dims,
                   theta 1e4) and proportional partial (global family: first
                   128 of 512 dims, theta 1e6, frequency denominator 512)
                   (pegainfer "Gemma 4" page, Architecture notes table and
                   bullets).
* ``attention`` -- naive, fully materialised masked softmax attention over
                   contiguous K/V, with the sliding window of the local family
                   and the single tied K/V head of the global family, plus the
                   rebuild of K from the compressed global record (Gewell
                   post, "the Why"; pegainfer "Gemma 4" page, intro and
                   Architecture notes).
* ``pool``      -- the library's documented in-page element layouts, decoded
                   back to contiguous K/V, and the per-family byte model
                   (pegainfer "Gemma 4" page, Scheduling: 16-token pages, one
                   pool per family).
* ``layers``    -- which layers of the hybrid stack are global (pegainfer
                   "Gemma 4" page, intro and Architecture notes).

Every function is pinned by ``tests/test_oracle_*.py`` (``-m "not gpu"``)
against values the pages print, closed forms, invariants and library
routines.  Parity unpinned: whether the real checkpoint pairs rotary dims as
rotate-half (this oracle) or interleaved; it does not affect attention parity
because the rotated K is stored.
"""

from . import codecs, rope, attention, pool, layers  # noqa: F401

__all__ = ["codecs", "rope", "attention", "pool", "layers"]
