"""Host page allocator (gw_alloc_*) against the oracle's pool model, and the
model against the pages' own numbers (CPU only; the library is loaded but
nothing touches a GPU)."""

import json
import os

import numpy as np
import pytest

from oracle import allocator as OA
from paged_hybrid_kv_amd import gw

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def reserve_rule(total, rows, window=1024):
    # the library's closed form of the local worst case
    return min(OA.pages_for(total), (rows + window + 13) // 16 + 1)


@pytest.mark.parametrize("window", [1024, 64, 17])
def test_local_reservation_is_the_worst_case(window):
    """The closed form equals the brute-force worst case over every step."""
    for total in (1, 15, 16, 17, 100, 1024, 1040, 3000):
        for rows in sorted({1, 2, 15, 16, 17, 511, 512, total}):
            if rows <= total:
                assert reserve_rule(total, rows, window) == OA.local_worst_case(total, rows, window), (total, rows)


def test_decode_window_spans_at_most_65_pages():
    # a 1024-token window over 16-token pages: 64 pages when aligned, 65 else
    assert OA.local_worst_case(8192, 1, 1024) == 65
    assert reserve_rule(8192, 1) == 65


def test_global_pool_is_slots_times_ceiling():
    """At the defaults (16 slots, 8192-token ceiling) the global pool that
    admits every slot at the ceiling is 16 x 512 pages; one page fewer and
    the sixteenth request waits."""
    slots = GOLD["decode_slots"]["value"]
    ceiling = GOLD["max_context"]["value"]
    assert GOLD["global_pool_rule"]["value"] == "slots x ceiling"
    need = slots * OA.pages_for(ceiling)
    assert need == 8192
    for pages, last in ((need, "admit"), (need - 1, "wait")):
        m = OA.PoolModel(slots, ceiling, 1024, 10 ** 6, pages)
        res = [m.admit(ceiling, 1)[0] for _ in range(slots)]
        assert res[:-1] == ["admit"] * (slots - 1) and res[-1] == last
    m = OA.PoolModel(slots, ceiling, 1024, 10 ** 6, need)
    for _ in range(slots):
        m.admit(ceiling, 1)
    assert m.admit(16, 1)[0] == "wait"          # past the slot count: waits


def test_refused_only_when_nothing_runs():
    m = OA.PoolModel(4, 8192, 1024, 100, 1000)
    assert m.admit(8193, 1)[0] == "refuse"      # past the ceiling
    assert m.admit(8000, 8000)[0] == "refuse"   # more local pages than the pool, nothing runs
    assert m.admit(100, 1)[0] == "admit"
    assert m.admit(8000, 8000)[0] == "wait"     # the same request waits while another runs


def _run(ops, args):
    """Apply ops to the library and the model side by side, comparing every
    decision, every table and the free counts."""
    slots, max_context, window, lp, gp = args
    A = gw.PageAllocator(*args)
    M = OA.PoolModel(*args, local_reserve=lambda t, r: reserve_rule(t, r, window))
    for op in ops:
        if op[0] == "admit":
            want = M.admit(op[1], op[2])
            try:
                got = A.admit(op[1], op[2])
                got = ("admit", got) if got >= 0 else ("wait", None)
            except gw.GwError as e:
                assert e.code == gw.GW_ERR_REFUSED
                got = ("refuse", None)
            assert got == want, op
        elif op[0] == "extend":
            A.extend(*op[1:])
            M.extend(*op[1:])
        else:
            A.release(op[1])
            M.release(op[1])
        lpt, gpt, lens = A.tables()
        ml, mg, mlens = M.tables()
        assert np.array_equal(lpt, np.array(ml)) and np.array_equal(gpt, np.array(mg)), op
        assert np.array_equal(lens, np.array(mlens))
        st = A.stats()
        assert st[:2] == (len(M.free["local"]), len(M.free["global"]))
        assert st[2:5] == (M.reserved("local"), M.reserved("global"), len(M.req))
        # validity: no page held twice within a family, all ids in range
        for t, n in ((lpt, lp), (gpt, gp)):
            held = t[t >= 0]
            assert len(np.unique(held)) == len(held) and (held < n).all()


@pytest.mark.parametrize("seed", range(6))
def test_random_runs_match_the_model(seed):
    rng = np.random.default_rng(seed)
    args = (4, 2048, 256, 90, 300)
    ops, live = [], {}
    M = OA.PoolModel(*args, local_reserve=lambda t, r: reserve_rule(t, r, 256))
    for _ in range(120):
        k = rng.integers(0, 10)
        if k < 3:
            total = int(rng.integers(1, 2300))
            rows = int(rng.integers(1, min(total, 600) + 1))
            op = ("admit", total, rows)
            res = M.admit(total, rows)
            if res[0] == "admit":
                live[res[1]] = [total, rows, 0, 0]
        elif k < 9 and live:
            s = int(rng.choice(sorted(live)))
            total, rows, L, fq = live[s]
            if L >= total:
                continue
            step = int(rng.integers(1, min(rows, total - L) + 1)) if L == 0 else int(rng.integers(1, min(rows, total - L) + 1))
            new_len = L + step
            first = max(fq, new_len - step)
            op = ("extend", s, new_len, first)
            M.extend(s, new_len, first)
            live[s] = [total, rows, new_len, first]
        elif live:
            s = int(rng.choice(sorted(live)))
            op = ("release", s)
            M.release(s)
            del live[s]
        else:
            continue
        ops.append(op)
    _run(ops, args)


def test_front_of_window_is_freed_and_global_is_not():
    A = gw.PageAllocator(1, 8192, 1024, 65, 512)
    s = A.admit(8192, 1)
    for L in range(1, 8193):
        A.extend(s, L, L - 1)
    lpt, gpt, lens = A.tables()
    assert lens[0] == 8192
    assert (gpt[0] >= 0).all()                           # all 512 global pages held
    held = np.nonzero(lpt[0] >= 0)[0]
    assert held[0] == (8191 - 1023) // 16 and held[-1] == 511
    assert A.stats()[0] == 65 - len(held)


@pytest.mark.parametrize("call,frag", [
    (lambda A: A.extend(0, 10, 0), "not active"),
    (lambda A: A.release(3), "not active"),
    (lambda A: A.admit(0, 1), "total_tokens"),
    (lambda A: A.admit(10, 11), "max_step_rows"),
])
def test_alloc_rejects(call, frag):
    A = gw.PageAllocator(2, 1024, 256, 100, 100)
    with pytest.raises(gw.GwError) as e:
        call(A)
    assert e.value.code == gw.GW_ERR_INVALID_ARG and frag in e.value.message


def test_extend_rejects_bad_steps():
    A = gw.PageAllocator(2, 1024, 256, 100, 100)
    s = A.admit(500, 64)
    A.extend(s, 100, 40)
    for args, frag in (((s, 99, 98), "new_len"), ((s, 501, 500), "new_len"), ((s, 120, 30), "first_query_pos"),
                       ((s, 300, 200), "max_step_rows")):
        with pytest.raises(gw.GwError) as e:
            A.extend(*args)
        assert frag in e.value.message
