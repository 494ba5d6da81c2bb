"""Page budget and page tables of the two families over a run of requests:
a plain model of the pool lifecycle.

Test infrastructure only (see ``oracle/__init__``).

pegainfer "Gemma 4" page, Scheduling:
* requests are admitted while the pools can hold them, up to the slot
  count; prompt + max_tokens is checked against the ceiling at admission;
* a request that cannot be admitted waits at the head of the queue and is
  refused only when nothing else is running (no pages can free up then);
* the two families have separate budgets: local layers free the front of
  the window past the window length, global layers free nothing while the
  request runs (their pool is slots x ceiling pages).

Readings where the pages leave a step open (each listed in the design notes):
* admission reserves the request's worst case in each family -- global, all
  of its pages; local, the most pages one step can touch: the pages from
  the window start of the step's first row to its last row;
* a local page is freed once it lies wholly before the window of the
  earliest row still to be queried;
* page ids are handed out lowest free id first (a rule of the library's own
  so that tables can be compared exactly).
"""

from __future__ import annotations

PAGE = 16


def pages_for(tokens: int) -> int:
    return -(-tokens // PAGE)


def local_worst_case(total: int, rows: int, window: int) -> int:
    """Most local pages a request holds at once: brute force over every step
    shape -- the rows p0 .. p0 + rows - 1 touch pages from the window start
    of p0 to the page of the last row."""
    best = 0
    for p0 in range(0, total):
        last = min(total - 1, p0 + rows - 1)
        lo = max(0, p0 - window + 1)
        best = max(best, last // PAGE - lo // PAGE + 1)
    return best


class PoolModel:
    def __init__(self, slots, max_context, window, local_pages, global_pages, local_reserve=None):
        self.slots, self.max_context, self.window = slots, max_context, window
        self.free = {"local": set(range(local_pages)), "global": set(range(global_pages))}
        self.size = {"local": local_pages, "global": global_pages}
        self.req = {}                       # slot -> dict
        # the local reservation rule; by default the brute-force worst case
        self.local_reserve = local_reserve or (lambda total, rows: local_worst_case(total, rows, window))

    def reserved(self, fam):
        return sum(r["res"][fam] for r in self.req.values())

    def admit(self, total, rows):
        """('admit', slot) | ('wait', None) | ('refuse', None)"""
        if total > self.max_context:
            return ("refuse", None)
        need = {"global": pages_for(total), "local": self.local_reserve(total, rows)}
        free_slots = [s for s in range(self.slots) if s not in self.req]
        fits = all(self.reserved(f) + need[f] <= self.size[f] for f in need)
        if free_slots and fits:
            s = free_slots[0]
            self.req[s] = {"total": total, "rows": rows, "len": 0, "res": need,
                           "pages": {"local": {}, "global": {}}}
            return ("admit", s)
        return ("refuse", None) if not self.req else ("wait", None)

    def _take(self, fam):
        i = min(self.free[fam])
        self.free[fam].remove(i)
        return i

    def extend(self, slot, new_len, first_query):
        r = self.req[slot]
        for fam in ("global", "local"):
            held = r["pages"][fam]
            lo = max(0, first_query - self.window + 1) // PAGE if fam == "local" else 0
            for lp in sorted(held):
                if lp < lo:
                    self.free[fam].add(held.pop(lp))
            for lp in range(lo, (new_len - 1) // PAGE + 1):
                if lp not in held:
                    held[lp] = self._take(fam)
            assert len(held) <= r["res"][fam], "a request outgrew its reservation"
        r["len"] = new_len

    def release(self, slot):
        r = self.req.pop(slot)
        for fam in ("global", "local"):
            self.free[fam].update(r["pages"][fam].values())

    def tables(self):
        n = pages_for(self.max_context)
        out = {}
        for fam in ("local", "global"):
            t = [[-1] * n for _ in range(self.slots)]
            for s, r in self.req.items():
                for lp, pp in r["pages"][fam].items():
                    t[s][lp] = pp
            out[fam] = t
        lens = [self.req[s]["len"] if s in self.req else 0 for s in range(self.slots)]
        return out["local"], out["global"], lens
