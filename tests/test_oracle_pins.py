"""Pins of the CPU reference (oracle) to things other than itself.

The pages print no worked example, so the reference is pinned by:
  * a brute-force model written separately (tests/brute.py) on thousands of
    tiny random scenarios,
  * the textbook least-recently-used cache (collections.OrderedDict) in the
    case of one selected row per call,
  * closed forms of special cases (no eviction, all pages ready),
  * a hand-worked trace,
  * library routines (numpy.unique) for the verify-block union,
  * the seeded payload's closed form for every gathered byte,
  * invariants after every step on the reduced workloads.
"""
from __future__ import annotations

from collections import OrderedDict

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import oracle as orc
from oracle.runner import OracleRun
from synth import Inputs, payload_np, tiny
from synth.gen import mix64_np
from tests.brute import BruteSource
from tests.helpers import new_row, one_request_source

TAIL, PAGE, HOT = 0, 1, 2


FRESH = 1 << 29  # hot-cache word of a row copied from host in the call


def word(place, idx):
    return (place << 30) | idx


# ----------------------------------------------------------------- payload


def test_splitmix64_published_vectors():
    # SplitMix64 seeded with 0: the first three outputs of the published generator
    got = mix64_np(np.array([0, 0x9E3779B97F4A7C15, 0x3C6EF372FE94F82A], dtype=np.uint64))
    assert [int(x) for x in got] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_c_filler_matches_numpy_closed_form():
    cfg = tiny(5)
    inp = Inputs(cfg)
    host = np.empty((cfg.n_req, inp.host_rows, cfg.R), dtype=np.uint8)
    inp.fill_host(0, host)
    for r in range(cfg.n_req):
        rows = np.nonzero(np.repeat(inp.host_valid[r], cfg.P)[:cfg.H])[0][::97]
        assert np.array_equal(host[r, rows], payload_np(0, r, rows, cfg.R, cfg.seed))
        bad = np.nonzero(np.repeat(inp.host_valid[r], cfg.P)[:cfg.H] == 0)[0]
        assert (host[r, bad] == 0xDB).all()


# ----------------------------------------------------------------- hand-worked trace


def test_hand_worked_trace():
    """H=8, P=4, T=2, B=2; page 0 ready at physical page 3, page 1 only on host.

    Derivation (one LRU tick per call; ties among equal stamps go to the lower
    slot; ascending missing rows take ascending victims):
      call 1, L=8, tail={6,7}: 7 tail slot 1; 1 page row 3*4+1=13; {4,5} miss
              -> slots 0,1; clock 1, stamps [1,1]
      append row 8 -> L=9, tail={7,8}
      call 2: {5,6} pending; 5 hits slot 1; 6 misses and takes slot 0 (the
              only slot not hit); clock 2, stamps [2,2], tags [6,5]
      call 3: 8 tail slot 0; 2 page row 14; 4 misses; both stamps 2 -> slot 0;
              clock 3, stamps [3,2], tags [4,5]
      call 4: {4,5,6} pending > B -> capacity error, nothing changes
      call 5: row 9 >= L -> range error, nothing changes
      call 6: 6 misses; least recent is slot 1 (stamp 2) -> tags [4,6],
              stamps [3,4], clock 4
    Hot-cache words of rows copied from host in the call carry the fresh flag.
    """
    src = one_request_source(H=8, P=4, T=2, B=2, page_map=[3, -1], host_valid=[0, 1])

    def call(sel):
        return src.resolve(np.array([sel], dtype=np.int32))

    loc, fills, fc, st = call([5, 1, 7, 4])
    assert st[0] == orc.OK
    assert loc[0].tolist() == [word(HOT, 1) | FRESH, word(PAGE, 13), word(TAIL, 1),
                               word(HOT, 0) | FRESH]
    assert fills[0, :fc[0]].tolist() == [[4, 0], [5, 1]]
    assert src.tag[0].tolist() == [4, 5] and src.stamp[0].tolist() == [1, 1] and src.clock[0] == 1

    assert src.append(new_row(src, 8))[0] == orc.OK and src.L[0] == 9
    loc, fills, fc, st = call([6, 5])
    assert loc[0].tolist() == [word(HOT, 0) | FRESH, word(HOT, 1)]
    assert fills[0, :fc[0]].tolist() == [[6, 0]]
    assert src.tag[0].tolist() == [6, 5] and src.stamp[0].tolist() == [2, 2]

    loc, fills, fc, st = call([4, 8, 2])
    assert loc[0].tolist() == [word(HOT, 0) | FRESH, word(TAIL, 0), word(PAGE, 14)]
    assert src.tag[0].tolist() == [4, 5] and src.stamp[0].tolist() == [3, 2] and src.clock[0] == 3

    loc, fills, fc, st = call([6, 5, 4])
    assert st[0] == orc.E_CAPACITY and fc[0] == 0 and (loc == orc.INVALID).all()
    assert src.tag[0].tolist() == [4, 5] and src.stamp[0].tolist() == [3, 2] and src.clock[0] == 3

    loc, fills, fc, st = call([9])
    assert st[0] == orc.E_RANGE and (loc == orc.INVALID).all() and src.clock[0] == 3

    loc, fills, fc, st = call([6])
    assert loc[0].tolist() == [word(HOT, 1) | FRESH]
    assert src.tag[0].tolist() == [4, 6] and src.stamp[0].tolist() == [3, 4] and src.clock[0] == 4

    # the hot cache now holds the host bytes of rows 4 and 6, the gather finds
    # them (with or without the fresh flag)
    out, gst = src.gather(0, np.array([[word(HOT, 0), word(HOT, 1) | FRESH, word(PAGE, 13),
                                        word(TAIL, 0)]], dtype=np.uint32))
    assert gst[0] == orc.OK
    assert np.array_equal(out[0], payload_np(0, 0, np.array([4, 6, 1, 8]), src.R, 7))


# ----------------------------------------------------------------- brute force


def _random_scenario(rng):
    P = int(rng.choice([1, 2, 3, 4, 8]))
    H = int(rng.integers(1, 40))
    T = int(rng.choice([0, 1, 2, 3, 5]))
    B = int(rng.integers(1, 7))
    n_pages = -(-H // P)
    full = H // P
    page_map = np.full(n_pages, -1, dtype=np.int32)
    ready = rng.random(full) < rng.random()
    page_map[:full][ready] = rng.permutation(int(ready.sum())) + int(rng.integers(0, 3))
    host_valid = np.where(page_map >= 0, rng.integers(0, 2, n_pages), 1).astype(np.uint8)
    if rng.random() < 0.1:  # break the residency invariant to reach the no-host-copy error
        host_valid[rng.integers(0, n_pages)] = 0
    return H, P, T, B, page_map, host_valid


def _brute_stats(stats, bst, bloc, bfills, R):
    """Add one resolve call's counters, derived from the brute model's
    outcome, to `stats` (keyed like orc.STAT_NAMES): every call counts; a
    failed call counts an error and nothing else; a good call counts its
    entries by place (hot-cache entries split by the fresh flag into hits and
    misses) and its fills, each of R host bytes (layer 0 is filled)."""
    stats["calls"] += 1
    if bst != 0:
        stats["error"] += 1
        return
    for place, idx in bloc:
        if place == 0:
            stats["tail"] += 1
        elif place == 1:
            stats["page"] += 1
        elif idx & FRESH:
            stats["miss"] += 1
        else:
            stats["hit"] += 1
    stats["fill"] += len(bfills)
    stats["host_bytes"] += len(bfills) * R


def _brute_residency_holds(bf, L):
    """Every imported row below L is in the tail, in a ready page or has a
    host copy (from the brute model's place sets)."""
    tail, ready = bf.tail_rows(), bf.ready_rows()
    return all(pos in tail or pos in ready or bf.host_valid[pos // bf.P]
               for pos in range(min(L, bf.H)))


@pytest.mark.parametrize("chunk", range(6))
def test_oracle_equals_brute_force(chunk):
    counts = {}
    broken = 0
    for seed in range(chunk * 300, chunk * 300 + 300):
        rng = np.random.default_rng(seed)
        H, P, T, B, page_map, host_valid = _random_scenario(rng)
        n_layers = int(rng.integers(1, 3))
        src = one_request_source(H, P, T, B, page_map, host_valid, R=16, n_layers=n_layers,
                                 max_new=12, seed=seed)
        bf = BruteSource(H, P, T, B, page_map, host_valid, n_layers=n_layers)
        stats = dict.fromkeys(orc.STAT_NAMES, 0)
        for _ in range(int(rng.integers(1, 12))):
            if rng.random() < 0.5 and src.L[0] < H + 12:
                assert src.append(new_row(src, int(src.L[0]), seed=seed))[0] == orc.OK
                bf.append()
            L = int(src.L[0])
            k = int(rng.integers(0, 9))
            sel = rng.integers(0, L, k)
            if k and rng.random() < 0.05:
                sel[rng.integers(0, k)] = rng.choice([-1, L, L + 3])
            loc, fills, fc, st = src.resolve(sel[None].astype(np.int32))
            bst, bloc, bfills = bf.resolve(sel.tolist())
            counts[bst] = counts.get(bst, 0) + 1
            _brute_stats(stats, bst, bloc, bfills, 16)
            assert dict(zip(orc.STAT_NAMES, src.stats.tolist())) == stats, seed
            assert st[0] == bst, (seed, sel)
            assert src.tag[0].tolist() == bf.tags(), seed
            assert src.stamp[0].tolist() == bf.stamps(), seed
            assert int(src.clock[0]) == bf.clock
            assert fills[0, :fc[0]].tolist() == [list(f) for f in bfills]
            if bst != 0:
                assert (loc == orc.INVALID).all()
                continue
            assert loc[0].tolist() == [word(p, i) for p, i in bloc]
            for l in range(1, n_layers):
                src.replay(l, fills, fc)
                bf.replay(l, bfills)
            for l in range(n_layers):
                out, gst = src.gather(l, loc)
                assert gst[0] == 0
                labels = [bf.label(l, p, i) for p, i in bloc]
                assert labels == sel.tolist()
                assert np.array_equal(out[0], payload_np(l, 0, np.array(labels, dtype=np.int64),
                                                         16, seed).reshape(k, 16))
        # the residency bit is set exactly when the scenario broke the
        # invariant for a row below L that is outside the tail
        holds = _brute_residency_holds(bf, int(src.L[0]))
        broken += not holds
        assert src.check()[0] == (0 if holds else 1), seed
    assert counts.get(0, 0) > 500 and counts.get(orc.E_CAPACITY, 0) > 10
    assert broken > 5


@settings(max_examples=400, deadline=None, derandomize=True, database=None)
@given(B=st.integers(1, 4), T=st.integers(0, 2), P=st.sampled_from([1, 2, 4]),
       H=st.integers(1, 64), data=st.data())
def test_oracle_equals_brute_force_hypothesis(B, T, P, H, data):
    """The same comparison with shapes and calls drawn by hypothesis (shrinks a
    failing case to a minimal one): B in 1..4, T in 0..2, P in {1, 2, 4},
    H <= 64, up to 20 calls of k <= 8 rows."""
    n_pages, full = -(-H // P), H // P
    ready = data.draw(st.lists(st.booleans(), min_size=full, max_size=full))
    page_map = np.full(n_pages, -1, dtype=np.int32)
    ids = iter(range(full))
    for p, rd in enumerate(ready):
        if rd:
            page_map[p] = next(ids)
    host_valid = np.where(page_map >= 0, 0, 1).astype(np.uint8)
    src = one_request_source(H, P, T, B, page_map, host_valid, R=16, n_layers=1, max_new=20,
                             seed=5)
    bf = BruteSource(H, P, T, B, page_map, host_valid, n_layers=1)
    stats = dict.fromkeys(orc.STAT_NAMES, 0)
    for _ in range(data.draw(st.integers(1, 20))):
        if data.draw(st.booleans()) and src.L[0] < H + 20:
            assert src.append(new_row(src, int(src.L[0]), seed=5))[0] == orc.OK
            bf.append()
        L = int(src.L[0])
        sel = data.draw(st.lists(st.integers(0, L - 1), max_size=8))
        loc, fills, fc, st_ = src.resolve(np.array([sel], dtype=np.int32).reshape(1, len(sel)))
        bst, bloc, bfills = bf.resolve(sel)
        _brute_stats(stats, bst, bloc, bfills, 16)
        assert dict(zip(orc.STAT_NAMES, src.stats.tolist())) == stats
        assert st_[0] == bst
        assert src.tag[0].tolist() == bf.tags() and src.stamp[0].tolist() == bf.stamps()
        assert int(src.clock[0]) == bf.clock
        assert fills[0, :fc[0]].tolist() == [list(f) for f in bfills]
        if bst == orc.OK:
            assert loc[0].tolist() == [word(p, i) for p, i in bloc]
        assert src.check()[0] == 0


# ----------------------------------------------------------------- invariant check


def test_check_reports_each_invariant_violation():
    """The state check returns the exact bit of each invariant a hand-built
    state breaks (1: a row below L that is in neither the tail nor a ready
    page and has no host copy; 2: a tag outside [-1, L) or held by two slots;
    4: a stamp newer than the clock), and 0 for states that keep them,
    including their edges (a page without host copy whose rows all sit in the
    tail, a tag of L - 1, a stamp equal to the clock)."""
    # H=16, P=4, T=4: tail rows 12..15 (page 3); pages 0 and 2 ready at
    # physical pages 1 and 0 without host copies; page 1 only on the host
    src = one_request_source(H=16, P=4, T=4, B=4, page_map=[1, -1, 0, -1],
                             host_valid=[0, 1, 0, 1], R=16)
    assert src.check().tolist() == [0]

    def mask():
        return int(src.check()[0])

    # residency: page 1 loses its host copy -> rows 4..7 are nowhere
    src.host_valid[0, 1] = 0
    assert mask() == 1
    src.host_valid[0, 1] = 1
    # page 3 without host copy and not ready, but every row in the tail
    src.host_valid[0, 3] = 0
    assert mask() == 0
    # one append moves row 12 out of the tail window: now it is nowhere
    assert src.append(new_row(src, 16))[0] == orc.OK
    assert mask() == 1
    src.host_valid[0, 3] = 1
    assert mask() == 0
    # a ready page released without a host copy
    src.page_map[0, 2] = -1
    assert mask() == 1
    src.page_map[0, 2] = 0

    L = int(src.L[0])
    src.clock[0] = 5
    src.tag[0] = [3, L - 1, -1, 9]
    src.stamp[0] = [5, 4, 0, 1]
    assert mask() == 0
    for bad in ([3, L, -1, 9], [3, L - 1, -2, 9], [3, 9, -1, 9], [7, L - 1, 7, 9]):
        src.tag[0] = bad
        assert mask() == 2, bad
    src.tag[0] = [3, L - 1, -1, 9]
    src.stamp[0] = [5, 6, 0, 1]
    assert mask() == 4
    src.stamp[0] = [5, 4, 0xFFFFFFFF, 1]   # an empty slot's stamp counts too
    assert mask() == 4
    # all three at once
    src.host_valid[0, 1] = 0
    src.tag[0] = [3, 3, -1, 9]
    assert mask() == 7


def test_check_residency_bit_on_a_partial_last_page():
    """A trailing partial page is never ready, so its rows need a host copy
    once they leave the tail."""
    src = one_request_source(H=14, P=4, T=2, B=2, page_map=[0, -1, -1, -1],
                             host_valid=[0, 1, 1, 1], R=16)
    assert src.check().tolist() == [0]
    src.host_valid[0, 3] = 0     # rows 12, 13: both in the tail (L = 14, T = 2)
    assert src.check().tolist() == [0]
    assert src.append(new_row(src, 14))[0] == orc.OK   # row 12 leaves the tail
    assert src.check().tolist() == [1]


# ----------------------------------------------------------------- textbook LRU


@pytest.mark.parametrize("B", [1, 2, 3, 5, 8])
def test_single_row_calls_are_textbook_lru(B):
    """One selected row per call: hits, misses and the resident set follow an
    OrderedDict LRU of capacity B exactly."""
    H = 64
    src = one_request_source(H=H, P=8, T=0, B=B, page_map=[-1] * 8, host_valid=[1] * 8, R=16)
    lru = OrderedDict()
    rng = np.random.default_rng(B)
    seq = rng.zipf(1.3, 600) % H
    for u in seq.tolist():
        loc, fills, fc, st = src.resolve(np.array([[u]], dtype=np.int32))
        assert st[0] == 0
        hit = u in lru
        if hit:
            lru.move_to_end(u)
        else:
            if len(lru) == B:
                lru.popitem(last=False)
            lru[u] = True
        assert (fc[0] == 0) == hit
        assert set(t for t in src.tag[0].tolist() if t >= 0) == set(lru)
        assert src.tag[0][loc[0, 0] & (FRESH - 1)] == u


# ----------------------------------------------------------------- special cases


def test_no_eviction_fills_slots_in_order():
    """B at least the number of distinct rows ever pending: nothing is evicted and
    the fills take slots 0, 1, 2, ... in order of (call, ascending row)."""
    H, B = 200, 256
    src = one_request_source(H=H, P=10, T=0, B=B, page_map=[-1] * 20, host_valid=[1] * 20, R=16)
    rng = np.random.default_rng(3)
    seen = []
    for _ in range(20):
        sel = rng.integers(0, H, 13)
        new = sorted(set(sel.tolist()) - set(seen))
        loc, fills, fc, st = src.resolve(sel[None].astype(np.int32))
        expect = [[u, len(seen) + i] for i, u in enumerate(new)]
        assert fills[0, :fc[0]].tolist() == expect
        seen += new
    assert src.tag[0, :len(seen)].tolist() == seen and (src.tag[0, len(seen):] == -1).all()


def test_all_pages_ready_means_no_hot_traffic():
    """Every complete page ready and every decoded row still in the tail: no
    pending rows, no fills, the clock still ticks once per call."""
    H, P, T = 256, 16, 8
    src = one_request_source(H=H, P=P, T=T, B=4, page_map=list(range(16)), host_valid=[0] * 16,
                             R=16)
    rng = np.random.default_rng(0)
    for call in range(1, T + 1):
        src.append(new_row(src, int(src.L[0])))
        loc, fills, fc, st = src.resolve(rng.integers(0, src.L[0], (1, 50)).astype(np.int32))
        assert st[0] == 0 and fc[0] == 0 and ((loc >> 30) < 2).all()
        assert src.clock[0] == call and (src.tag[0] == -1).all()


def test_error_paths_commit_nothing_and_spare_other_requests():
    cfg = tiny(3)
    inp = Inputs(cfg)
    run = OracleRun(inp)
    run.step(0)
    src = run.src
    before = src.snapshot()
    L = int(src.L[0])
    sel = inp.selections(1)[:, 0, :].copy()
    sel[0, 5] = L               # request 0: out of range
    sel[1, :] = np.arange(cfg.k)  # request 1: fine (rows 0..k-1)
    host_valid_backup = src.host_valid.copy()
    # request 2: a not-ready page without host copy (breaks the residency invariant)
    pg = int(np.nonzero(src.page_map[2][: cfg.H // cfg.P] < 0)[0][0])
    src.host_valid[2, pg] = 0
    sel[2, 0] = pg * cfg.P
    # request 3: more distinct pending rows than B
    sel3 = np.nonzero(np.repeat(src.page_map[3], cfg.P)[:cfg.H] < 0)[0][: cfg.B + 1]
    wide = np.full((cfg.n_req, cfg.B + 1), 0, dtype=np.int32)
    wide[:, : cfg.k] = sel
    wide[3] = sel3
    count = np.full(cfg.n_req, cfg.k, dtype=np.int32)
    count[3] = cfg.B + 1
    loc, fills, fc, st = src.resolve(wide, count=count)
    assert st.tolist()[:4] == [orc.E_RANGE, orc.OK, orc.E_NO_HOST_COPY, orc.E_CAPACITY]
    for r in (0, 2, 3):
        assert (loc[r, : count[r]] == orc.INVALID).all() and fc[r] == 0
        assert np.array_equal(src.tag[r], before["tag"][r])
        assert np.array_equal(src.stamp[r], before["stamp"][r])
        assert src.clock[r] == before["clock"][r]
        assert np.array_equal(src.hot[0][r], before["hot"][0][r])
    assert src.clock[1] == before["clock"][1] + 1 and st[4] == 0
    src.host_valid[:] = host_valid_backup


def test_clock_wrap_is_a_state_error():
    src = one_request_source(H=8, P=4, T=0, B=2, page_map=[-1, -1], host_valid=[1, 1])
    src.clock[0] = 0xFFFFFFFF
    loc, fills, fc, st = src.resolve(np.array([[1]], dtype=np.int32))
    assert st[0] == orc.E_STATE and (src.tag[0] == -1).all()


def test_empty_selection_only_ticks():
    src = one_request_source(H=8, P=4, T=2, B=2, page_map=[-1, -1], host_valid=[1, 1])
    loc, fills, fc, st = src.resolve(np.zeros((1, 0), dtype=np.int32))
    assert st[0] == 0 and fc[0] == 0 and src.clock[0] == 1


# ----------------------------------------------------------------- order and duplicates


def test_permutation_and_duplicate_invariance():
    cfg = tiny(2)
    inp = Inputs(cfg)
    a, b = OracleRun(inp), OracleRun(inp)
    rng = np.random.default_rng(11)
    for s in range(cfg.steps):
        sel = inp.selections(s)
        perm = rng.permutation(sel.shape[2])
        dup = np.concatenate([sel[:, :, perm], sel[:, :, :20]], axis=2)
        ra = a.step(s, sels=[sel])["groups"][0]
        rb = b.step(s, sels=[dup])["groups"][0]
        assert np.array_equal(a.src.tag, b.src.tag) and np.array_equal(a.src.stamp, b.src.stamp)
        assert np.array_equal(ra["loc"][:, perm], rb["loc"][:, : len(perm)])
        assert np.array_equal(ra["loc"][:, :20], rb["loc"][:, len(perm):])
        assert np.array_equal(ra["fills"], rb["fills"])


def test_union_equals_concatenation_and_numpy_unique():
    """Resolving the union of a verify block gives the same state and the same
    location per row as resolving all queries' rows in any order."""
    cfg = tiny(4)
    inp = Inputs(cfg)
    a, b = OracleRun(inp), OracleRun(inp)
    rng = np.random.default_rng(5)
    for s in range(cfg.steps):
        sel = inp.selections(s)
        ra = a.step(s, sels=[sel])["groups"][0]
        flat = sel.reshape(cfg.n_req, -1)
        perm = rng.permutation(flat.shape[1])
        b.src.append(inp.new_rows(s))
        loc_b, fills_b, fc_b, st_b = b.src.resolve(flat[:, perm])
        for l in range(1, cfg.payload_layers):
            b.src.replay(l, fills_b, fc_b)
        assert (st_b == 0).all() and (ra["status"] == 0).all()
        assert np.array_equal(a.src.tag, b.src.tag) and np.array_equal(a.src.stamp, b.src.stamp)
        for r in range(cfg.n_req):
            u = np.unique(flat[r])
            n = ra["union_count"][r]
            assert n == len(u) and np.array_equal(ra["union"][r, :n], u)
            assert np.array_equal(ra["union"][r][ra["map"][r]], sel[r])
            per_row = dict(zip(flat[r, perm].tolist(), loc_b[r].tolist()))
            assert [per_row[x] for x in u.tolist()] == ra["loc"][r, :n].tolist()


# ----------------------------------------------------------------- reduced workloads


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_reduced_workload_invariants_and_bytes(c):
    cfg = tiny(c)
    inp = Inputs(cfg)
    run = OracleRun(inp)
    src = run.src
    for s in range(cfg.steps):
        prev_stamp = src.stamp.copy()
        res = run.step(s)
        assert (res["append_status"] == 0).all()
        L = inp.length_at(s)
        for g, rec in enumerate(res["groups"]):
            assert (rec["status"] == 0).all()
            rows = rec["union"] if cfg.q > 1 else rec["sel"][:, 0, :]
            count = rec["count"] if rec["count"] is not None else np.full(cfg.n_req, rows.shape[1])
            for r in range(cfg.n_req):
                n = count[r]
                pos = rows[r, :n]
                loc = rec["loc"][r, :n]
                place = loc >> 30
                # step 1 closed form: tail window, then complete ready pages
                in_tail = pos >= max(0, L - cfg.T)
                pm = src.page_map[r]
                full = pos < (cfg.H // cfg.P) * cfg.P
                ready = full & (pm[np.minimum(pos // cfg.P, len(pm) - 1)] >= 0)
                expect = np.where(in_tail, 0, np.where(ready, 1, 2))
                assert np.array_equal(place, expect)
                # hit slots are not victims; all referenced slots carry the new tick
                fslots = rec["fills"][r, : rec["fill_count"][r], 1]
                hot_slots = np.unique(loc[place == 2] & (FRESH - 1))
                hit_slots = np.setdiff1d(hot_slots, fslots)
                tick = src.clock[r] - (cfg.groups - 1 - g)   # this group's tick
                if g == cfg.groups - 1:
                    assert (src.stamp[r, hot_slots] == tick).all()
                else:  # later groups of the step may only refresh a stamp
                    assert (src.stamp[r, hot_slots] >= tick).all()
                if cfg.groups == 1:
                    assert (prev_stamp[r, fslots] < tick).all()
                assert len(np.intersect1d(hit_slots, fslots)) == 0
                # every gathered byte is the payload of the selected position
                for l, out in enumerate(rec["out"]):
                    assert np.array_equal(out[r, :n], payload_np(l, r, pos, cfg.R, cfg.seed))
        assert (src.check() == 0).all()


# ----------------------------------------------------------------- regression fixture


def test_golden_regression_fixture():
    """The oracle still produces the stored trace (tests/golden/make_golden.py)."""
    import json
    import os

    from tests.golden.make_golden import run
    path = os.path.join(os.path.dirname(__file__), "golden", "lru_trace_small.json")
    fx = json.load(open(path))
    assert run(fx) == fx["expected"]
    statuses = {e["status"] for e in fx["expected"]}
    assert orc.E_CAPACITY in statuses and orc.OK in statuses
