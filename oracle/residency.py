"""Residency policy of the optional pool: the reference.

TEST INFRASTRUCTURE ONLY: tests and the benchmark's scenario checks use it;
the product path never imports it.  It shares no code with the GPU library's
policy (a separate C++ implementation).

Follows "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
Hierarchy", section "How it works":
  * paragraph "Memory split": whole pages of the history a request was
    admitted with may be held as optional capacity that can be taken back,
    beside the reserve that admissions use (the pool holds required,
    optional and reserve pages);
  * paragraph "Reclamation and refill": when an admission needs more pages
    than are free, requests give up all their optional pages, one request at
    a time in reclaim order, until the shortfall is met, and the requests
    after that keep theirs; when even all optional pages would not be enough
    the admission waits; refill brings pages back a bounded number at a
    time, visiting requests in turn.

Readings where the pages are silent:
  * the reclaim order is the caller's (a list of request ids);
  * an admission first uses free pages; only the remainder is a deficit, and
    every ready complete page of a taken request is released, in ascending
    page order;
  * physical pages are handed out lowest id first; an admission reserves the
    lowest free ids and gives them back when it drains;
  * refill brings back the pages reclamation took (the evidence section's
    load-step experiment: residency "repopulates as requests drain"); pages
    that were not ready at admission stay as admission left them;
  * refill visits requests cyclically from a cursor kept between calls; each
    visit gives the request its lowest-index reclaimed page not yet back; it
    stops after `bound` pages, when no free page is left, or when a whole
    cycle finds nothing; the cursor then points after the last request
    served.
The device side of each decision (host backup of a page without a host copy,
then release; host rows into the pool, then publish) is orc_reclaim_pages and
orc_restore_pages in kvr_oracle.c.
"""
from __future__ import annotations

import bisect


class ResidencyPolicy:
    def __init__(self, page_map, n_complete: int, pool_pages: int):
        """page_map: [n_req][n_pages] physical page or -1 (only the first
        n_complete pages of each request may be optional)."""
        self.n_req = len(page_map)
        self.n_complete = int(n_complete)
        self.ready = [[int(page_map[r][p]) for p in range(self.n_complete)]
                      for r in range(self.n_req)]
        used = {ph for row in self.ready for ph in row if ph >= 0}
        self.free = sorted(set(range(int(pool_pages))) - used)
        self.taken = [[] for _ in range(self.n_req)]  # reclaimed, not yet back
        self.reserved = {}
        self.next_handle = 0
        self.cursor = 0

    def admit(self, need: int, order):
        """An admission needing `need` physical pages.  Returns (True, the
        (request, page) list to reclaim, handle) or (False, [], -1) when the
        shortfall is larger than all optional pages together (nothing changes)."""
        assert need >= 0
        deficit = need - len(self.free)
        plan = []
        if deficit > 0:
            for r in order:
                if deficit <= 0:
                    break
                pages = [p for p in range(self.n_complete) if self.ready[r][p] >= 0]
                plan += [(r, p) for p in pages]
                deficit -= len(pages)
            if deficit > 0:
                return False, [], -1
            for r, p in plan:
                bisect.insort(self.free, self.ready[r][p])
                self.ready[r][p] = -1
                bisect.insort(self.taken[r], p)
        mine, self.free = self.free[:need], self.free[need:]
        handle = self.next_handle
        self.next_handle += 1
        self.reserved[handle] = mine
        return True, plan, handle

    def release(self, handle: int) -> None:
        """The admission drained: its reserved pages are free again."""
        for ph in self.reserved.pop(handle):
            bisect.insort(self.free, ph)

    def refill(self, bound: int):
        """Bounded round-robin refill of reclaimed pages.  Returns the
        (request, page, physical page) list to restore."""
        placed = []
        idle = 0
        r = self.cursor
        while len(placed) < bound and self.free and idle < self.n_req:
            if self.taken[r]:
                p = self.taken[r].pop(0)
                ph = self.free.pop(0)
                self.ready[r][p] = ph
                placed.append((r, p, ph))
                idle = 0
                self.cursor = (r + 1) % self.n_req
            else:
                idle += 1
            r = (r + 1) % self.n_req
        return placed

    def counts(self):
        """(free pages, ready pages, reserved pages)."""
        ready = sum(1 for row in self.ready for ph in row if ph >= 0)
        return len(self.free), ready, sum(len(v) for v in self.reserved.values())
