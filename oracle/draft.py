"""Drafter visible-window ring: the reference.

TEST INFRASTRUCTURE ONLY: tests use it; the product path never imports it.
It shares no code with the GPU library.

Follows "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
Hierarchy", section "How it works", paragraph "Speculative state": the
drafter stores just the rows it can still see, in a ring.

Readings where the page is silent:
  * a request's drafter rows are numbered by position 0, 1, 2, ...; `length`
    counts the rows appended and kept; the visible window is the last
    min(W, length) positions;
  * the ring holds capacity C >= W rows at slot position mod C, so that up to
    C - W drafted, not yet verified rows can be dropped again: a rollback to
    a shorter length (the accepted prefix) is allowed while every row of the
    window it leaves visible is still in its slot, i.e. no later position
    (kept or dropped) has been written over it: for a length of at least
    (the highest position ever written + 1) - (C - W); anything shorter is an
    error and changes nothing;
  * an append of a rows per request writes positions length .. length+a-1;
  * the window gather writes the visible rows in position order, oldest
    first; rows past the window's length are left untouched.
"""
from __future__ import annotations

import numpy as np

OK, E_RANGE = 0, -2


class DraftRing:
    def __init__(self, n_req: int, window: int, capacity: int, row_bytes: int):
        assert 1 <= window <= capacity
        self.n_req, self.W, self.C, self.R = n_req, window, capacity, row_bytes
        self.ring = np.zeros((n_req, capacity, row_bytes), dtype=np.uint8)
        self.length = np.zeros(n_req, dtype=np.int64)
        self.high = np.zeros(n_req, dtype=np.int64)  # highest position ever written + 1

    def append(self, rows: np.ndarray, req_ids=None) -> None:
        """rows: uint8 [n][a][R]: a new rows for each listed request."""
        req = range(self.n_req) if req_ids is None else req_ids
        for i, r in enumerate(req):
            for t in range(rows.shape[1]):
                pos = int(self.length[r]) + t
                self.ring[r, pos % self.C] = rows[i, t]
            self.length[r] += rows.shape[1]
            self.high[r] = max(self.high[r], self.length[r])

    def rollback(self, new_length, req_ids=None) -> np.ndarray:
        """Keep the first new_length[i] rows.  Returns a status per entry."""
        req = list(range(self.n_req)) if req_ids is None else list(req_ids)
        status = np.zeros(len(req), dtype=np.int32)
        for i, r in enumerate(req):
            keep = int(new_length[i])
            lo = int(self.high[r]) - (self.C - self.W)
            if keep < max(lo, 0) or keep > self.length[r]:
                status[i] = E_RANGE
                continue
            self.length[r] = keep
        return status

    def window(self, out: np.ndarray, req_ids=None) -> np.ndarray:
        """out: uint8 [n][W][R]; returns the visible row count per entry."""
        req = list(range(self.n_req)) if req_ids is None else list(req_ids)
        vis = np.zeros(len(req), dtype=np.int32)
        for i, r in enumerate(req):
            L = int(self.length[r])
            first = max(0, L - self.W)
            for t, pos in enumerate(range(first, L)):
                out[i, t] = self.ring[r, pos % self.C]
            vis[i] = L - first
        return vis
