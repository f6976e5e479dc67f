"""Pins of the residency reference (oracle/residency.py and the page
reclaim/restore of oracle/kvr_oracle.c) against facts fixed independently of
it: the payload closed form, the invariant that no row is ever without both
a ready page and a host backup, a hand-worked admission and refill, and properties the pages'
paragraph "Reclamation and refill" fixes (whole requests in reclaim order,
the deficit covered and no more requests than needed, bounded round-robin).
CPU only."""
from __future__ import annotations

import numpy as np
import pytest

from oracle.oracle import E_ARG, E_NO_HOST_COPY, E_RANGE, E_STATE, OK
from oracle.residency import ResidencyPolicy
from oracle.runner import OracleRun
from synth import Inputs, payload_np, tiny


def _run(c=2, spare=6, **kw):
    cfg = tiny(c).with_(pool_spare=spare, **kw)
    inputs = Inputs(cfg, max_new=cfg.steps + 2)
    return cfg, inputs, OracleRun(inputs)


def _page_rows(cfg, p):
    return np.arange(p * cfg.P, (p + 1) * cfg.P)


def test_reclaim_backs_up_then_releases():
    cfg, inputs, run = _run()
    src = run.src
    r = 1
    ready = np.nonzero(src.page_map[r] >= 0)[0][:3]
    phys = src.page_map[r, ready].copy()
    assert (src.host_valid[r, ready] == 0).all()  # resident-first: no host copy yet
    req = np.full(len(ready) + 1, r)
    page = np.concatenate([ready, ready[:1]])  # a repeat of the first entry
    freed, st = src.reclaim_pages(req, page)
    assert (st == OK).all()
    assert list(freed) == list(phys) + [-1]
    assert (src.page_map[r, ready] == -1).all() and (src.host_valid[r, ready] == 1).all()
    for l in range(cfg.payload_layers):
        for p in ready:
            rows = _page_rows(cfg, p)
            assert np.array_equal(src.host[l][r, rows], payload_np(l, r, rows, cfg.R, cfg.seed))
    assert (src.check() == 0).all()
    # a page that is not ready: nothing happens
    freed, st = src.reclaim_pages([r], [ready[0]])
    assert freed[0] == -1 and st[0] == OK
    freed, st = src.reclaim_pages([cfg.n_req, 0], [0, cfg.n_pages])
    assert list(st) == [E_ARG, E_ARG] and list(freed) == [-1, -1]
    # corrupt map entries (an incomplete page marked ready, a physical page
    # outside the pool) are refused and nothing moves
    part = cfg.H // cfg.P
    assert cfg.H % cfg.P != 0
    src.page_map[0, part] = 0
    q = int(np.nonzero(src.page_map[2] >= 0)[0][0])
    src.page_map[2, q] = cfg.pool_pages
    host0 = [h.copy() for h in src.host]
    freed, st = src.reclaim_pages([0, 2], [part, q])
    assert list(st) == [E_STATE, E_STATE] and list(freed) == [-1, -1]
    assert src.page_map[0, part] == 0 and src.page_map[2, q] == cfg.pool_pages
    assert all(np.array_equal(a, b) for a, b in zip(host0, src.host))


def test_restore_fills_the_pool_then_publishes():
    cfg, inputs, run = _run()
    src = run.src
    spare = np.nonzero(inputs.owner_req < 0)[0]
    r = 0
    not_ready = np.nonzero(src.page_map[r, :cfg.H // cfg.P] < 0)[0][:2]
    st = src.restore_pages([r, r], not_ready, spare[:2])
    assert (st == OK).all()
    assert list(src.page_map[r, not_ready]) == list(spare[:2])
    for l in range(cfg.payload_layers):
        for p, ph in zip(not_ready, spare[:2]):
            assert np.array_equal(src.pool[l][ph], payload_np(l, r, _page_rows(cfg, p), cfg.R, cfg.seed))
    assert (src.check() == 0).all()


def test_restore_errors_in_precedence():
    cfg, inputs, run = _run()
    src = run.src
    spare = [int(x) for x in np.nonzero(inputs.owner_req < 0)[0]]
    nr = [int(p) for p in np.nonzero(src.page_map[2, :cfg.H // cfg.P] < 0)[0]]
    rd = int(np.nonzero(src.page_map[2] >= 0)[0][0])
    partial = cfg.H // cfg.P  # tiny(2) has a trailing partial page
    assert cfg.H % cfg.P != 0
    before = src.page_map.copy()
    req = [2, 2, 2, 2, 2, 5, 2]
    page = [partial, nr[0], nr[0], nr[1], rd, 0, nr[2]]
    phys = [spare[0], spare[1], spare[2], spare[1], spare[3], spare[4], cfg.pool_pages]
    st = src.restore_pages(req, page, phys)
    # incomplete page; ok; same page again; same physical page again; already
    # ready; request out of range; physical page outside the pool
    assert list(st) == [E_ARG, OK, E_ARG, E_ARG, E_STATE, E_ARG, E_RANGE]
    after = src.page_map.copy()
    before[2, nr[0]] = spare[1]
    assert np.array_equal(after, before)
    # no host copy: a ready page that lost its map entry by corruption
    src.page_map[2, rd] = -1
    assert src.restore_pages([2], [rd], [spare[5]])[0] == E_NO_HOST_COPY


def test_resolution_after_reclaim_reads_host_copies():
    """Rows of reclaimed pages (backed up by the reclaim) resolve from the hot
    cache or host memory and gather the payload closed form."""
    cfg, inputs, run = _run(c=2, spare=0)
    src = run.src
    for s in range(2):
        run.step(s)
    reqs = [0, 2]
    plan = [(r, int(p)) for r in reqs for p in np.nonzero(src.page_map[r] >= 0)[0]]
    freed, st = src.reclaim_pages([r for r, _ in plan], [p for _, p in plan])
    assert (st == OK).all() and (freed >= 0).all()
    for s in range(2, cfg.steps):
        out = run.step(s)
        assert (src.check() == 0).all()
        rec = out["groups"][0]
        assert (rec["status"] == OK).all()
        sel = rec["sel"][:, 0, :]
        for r in range(cfg.n_req):
            for l in range(cfg.payload_layers):
                assert np.array_equal(rec["out"][l][r], payload_np(l, r, sel[r], cfg.R, cfg.seed))
        pm = src.page_map
        assert (pm[reqs] == -1).all()


def test_policy_hand_worked():
    # 3 requests, 4 complete pages each, pool of 10 physical pages
    pm = [[3, -1, 7, 0], [-1, -1, -1, -1], [5, 1, -1, 2]]
    pol = ResidencyPolicy(pm, 4, 10)
    assert pol.free == [4, 6, 8, 9]
    # needs 3: free pages cover it; the lowest free ids are reserved
    ok, plan, h0 = pol.admit(3, [0, 1, 2])
    assert ok and plan == [] and pol.reserved[h0] == [4, 6, 8] and pol.free == [9]
    # needs 4 with 1 free: deficit 3; request 1 has no ready page, request 0
    # (3 pages) covers it, request 2 keeps its pages
    ok, plan, h1 = pol.admit(4, [1, 0, 2])
    assert ok and plan == [(0, 0), (0, 2), (0, 3)]
    assert pol.reserved[h1] == [0, 3, 7, 9] and pol.free == []
    # needs 5 with 0 free: request 2's 3 pages cannot cover it: wait
    ok, plan, h2 = pol.admit(5, [0, 1, 2])
    assert not ok and plan == [] and h2 == -1 and pol.counts() == (0, 3, 7)
    # the first admission drains; refill brings request 0's pages back, 2 now
    pol.release(h0)
    assert pol.free == [4, 6, 8]
    assert pol.refill(2) == [(0, 0, 4), (0, 2, 6)]
    assert pol.cursor == 1
    assert pol.refill(5) == [(0, 3, 8)]
    assert pol.cursor == 1 and pol.free == []
    # page 1 of request 0 and all of request 1 were never ready: not refilled
    pol.release(h1)
    assert pol.refill(3) == [] and pol.free == [0, 3, 7, 9]
    # needs 8 with 4 free: deficit 4: request 2 (3 pages), then request 0
    ok, plan, h3 = pol.admit(8, [2, 0])
    assert ok and plan == [(2, 0), (2, 1), (2, 3), (0, 0), (0, 2), (0, 3)]
    assert pol.reserved[h3] == list(range(8)) and pol.free == [8, 9]
    pol.release(h3)
    # round robin from the cursor (request 1, nothing to bring back):
    # request 2, request 0, request 2, request 0
    assert pol.refill(4) == [(2, 0, 0), (0, 0, 1), (2, 1, 2), (0, 2, 3)]
    assert pol.cursor == 1
    assert pol.counts() == (6, 4, 0)


@pytest.mark.parametrize("seed", range(40))
def test_policy_properties(seed):
    rng = np.random.default_rng(seed)
    n_req, n_complete = int(rng.integers(1, 7)), int(rng.integers(1, 9))
    pool = int(rng.integers(n_complete, n_req * n_complete + 12))
    perm = rng.permutation(pool)
    pm = np.full((n_req, n_complete), -1, dtype=np.int64)
    k = 0
    for r in range(n_req):
        for p in range(n_complete):
            if k < pool and rng.random() < 0.5:
                pm[r, p] = perm[k]
                k += 1
    pol = ResidencyPolicy(pm, n_complete, pool)
    handles = []
    back = [set() for _ in range(n_req)]  # reclaimed pages not yet refilled
    for _ in range(30):
        free0 = list(pol.free)
        ready0 = [list(row) for row in pol.ready]
        op = rng.integers(0, 3)
        if op == 0:
            need = int(rng.integers(0, pool // 2 + 2))
            order = [int(x) for x in rng.permutation(n_req)]
            ok, plan, h = pol.admit(need, order)
            ready_of = [sum(ph >= 0 for ph in ready0[r]) for r in range(n_req)]
            deficit = need - len(free0)
            if deficit <= 0:
                assert ok and plan == []
            elif deficit > sum(ready_of):
                assert not ok and pol.free == free0 and pol.ready == ready0
                continue
            else:
                # whole requests, in reclaim order, the shortest prefix that covers
                taken = []
                for r, p in plan:
                    if not taken or taken[-1] != r:
                        taken.append(r)
                prefix = [r for r in order if ready_of[r] > 0]
                assert taken == prefix[:len(taken)]
                got = sum(ready_of[r] for r in taken)
                assert got >= deficit and got - ready_of[taken[-1]] < deficit
                assert plan == [(r, p) for r in taken for p in range(n_complete) if ready0[r][p] >= 0]
            for r, p in plan:
                back[r].add(p)
            handles.append(h)
            pool_after = sorted(free0 + [ready0[r][p] for r, p in plan])
            assert pol.reserved[h] == pool_after[:need] and pol.free == pool_after[need:]
        elif op == 1 and handles:
            h = handles.pop(int(rng.integers(0, len(handles))))
            returned = pol.reserved[h]
            pol.release(h)
            assert pol.free == sorted(free0 + returned)
        else:
            bound = int(rng.integers(0, 6))
            cur = pol.cursor
            placed = pol.refill(bound)
            assert len(placed) <= bound
            assert [ph for _, _, ph in placed] == free0[:len(placed)]
            # only reclaimed pages come back, each request's lowest first
            served = [r for r, _, _ in placed]
            for r in range(n_req):
                got = [p for rr, p, _ in placed if rr == r]
                assert got == sorted(back[r])[:len(got)]
                back[r] -= set(got)
            eligible = [r for r in range(n_req) if any(rr == r for rr, _, _ in placed)
                        or back[r]]
            # round robin from the cursor: the first served request is the
            # first eligible one from the cursor; counts differ by at most one
            # among requests that still had pages to bring back
            if served:
                assert served[0] == next(r for r in [(cur + i) % n_req for i in range(n_req)]
                                         if r in eligible)
                counts = [served.count(r) for r in range(n_req)]
                still = [r for r in eligible if back[r]]
                if still:
                    assert max(counts) - min(counts[r] for r in still) <= 1
            if len(placed) < bound:
                assert not pol.free or not any(back)
        f, rd, rs = pol.counts()
        assert f + rd + rs == pool
        used = [ph for row in pol.ready for ph in row if ph >= 0]
        assert len(set(used)) == len(used) and not set(used) & set(pol.free)
