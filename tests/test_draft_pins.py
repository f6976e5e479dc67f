"""Pins of the drafter visible-window ring reference (oracle/draft.py): the
window against the payload closed form and against a plain list model that
keeps every row, across appends, wrap-around and rollbacks.  CPU only."""
from __future__ import annotations

import numpy as np
import pytest

from oracle.draft import E_RANGE, OK, DraftRing
from synth import payload_np

R = 32
SEED = 4242


def rows_for(r, positions, version):
    # a rolled-back position gets different bytes when drafted again
    return payload_np(200 + version, r, np.asarray(positions), R, SEED)


def test_window_is_the_last_w_rows_in_order():
    ring = DraftRing(n_req=2, window=5, capacity=8, row_bytes=R)
    pos = [0, 0]
    for a in (3, 4, 1, 6):
        rows = np.stack([rows_for(r, range(pos[r], pos[r] + a), 0) for r in range(2)])
        ring.append(rows)
        pos = [p + a for p in pos]
        out = np.zeros((2, 5, R), dtype=np.uint8)
        vis = ring.window(out)
        for r in range(2):
            first = max(0, pos[r] - 5)
            assert vis[r] == pos[r] - first
            assert np.array_equal(out[r, :vis[r]], rows_for(r, range(first, pos[r]), 0))


def test_rollback_limits():
    ring = DraftRing(n_req=1, window=4, capacity=6, row_bytes=R)
    ring.append(rows_for(0, range(10), 0)[None])
    # the ring holds positions 4..9: a length of 7 would show 3..6, and 3 is
    # gone; 8 shows 4..7
    assert ring.rollback([7]).tolist() == [E_RANGE] and ring.length[0] == 10
    assert ring.rollback([8]).tolist() == [OK] and ring.length[0] == 8
    assert ring.rollback([9]).tolist() == [E_RANGE]         # longer than kept
    ring.append(rows_for(0, range(8, 10), 1)[None])          # 8, 9 drafted again
    assert ring.length[0] == 10
    out = np.zeros((1, 4, R), dtype=np.uint8)
    assert ring.window(out).tolist() == [4]
    assert np.array_equal(out[0, :2], rows_for(0, range(6, 8), 0))
    assert np.array_equal(out[0, 2:], rows_for(0, range(8, 10), 1))
    assert ring.rollback([8]).tolist() == [OK]
    assert ring.window(out).tolist() == [4]
    assert np.array_equal(out[0], rows_for(0, range(4, 8), 0))
    # a dropped row still took its slot: after 8 is drafted again and dropped,
    # ... positions 2, 3 (slots of 8, 9) stay gone
    ring.append(rows_for(0, [8], 2)[None])
    assert ring.rollback([7]).tolist() == [E_RANGE]


@pytest.mark.parametrize("seed", range(30))
def test_ring_equals_list_model(seed):
    rng = np.random.default_rng(seed)
    n_req = int(rng.integers(1, 4))
    W = int(rng.integers(1, 7))
    C = W + int(rng.integers(0, 6))
    ring = DraftRing(n_req, W, C, R)
    model = [[] for _ in range(n_req)]  # every kept row
    high = [0] * n_req                  # highest position ever written + 1
    version = 0
    for _ in range(25):
        version += 1
        if rng.random() < 0.6:
            a = int(rng.integers(1, 5))
            rows = np.stack([rows_for(r, range(len(model[r]), len(model[r]) + a), version)
                             for r in range(n_req)])
            ring.append(rows)
            for r in range(n_req):
                model[r] += list(rows[r])
                high[r] = max(high[r], len(model[r]))
        else:
            keep = [int(rng.integers(0, len(m) + 1)) for m in model]
            st = ring.rollback(keep)
            for r in range(n_req):
                # the window [keep - W, keep) must not have been overwritten
                # by any position written since (kept or dropped)
                ok = keep[r] >= max(0, high[r] - (C - W))
                assert st[r] == (OK if ok else E_RANGE)
                if ok:
                    model[r] = model[r][:keep[r]]
        out = np.zeros((n_req, W, R), dtype=np.uint8)
        vis = ring.window(out)
        for r in range(n_req):
            want = model[r][-W:] if model[r] else []
            assert vis[r] == len(want)
            for t, row in enumerate(want):
                assert np.array_equal(out[r, t], row)
