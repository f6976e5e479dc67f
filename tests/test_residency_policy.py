"""The library's host-side residency policy (kvr_residency_*, C++) makes the
same decisions as the reference policy (oracle/residency.py) over random
sequences of admissions, drains and refills, and rejects bad arguments.
Host logic only: no GPU is needed."""
from __future__ import annotations

import numpy as np
import pytest

from hierarchical_sparse_kv_resolve_amd import kvr
from oracle.residency import ResidencyPolicy


def _scenario(seed):
    rng = np.random.default_rng(seed)
    n_req, n_complete = int(rng.integers(1, 9)), int(rng.integers(1, 12))
    n_pages = n_complete + int(rng.integers(0, 2))  # maybe a trailing partial page
    pool = int(rng.integers(n_complete, n_req * n_complete + 16))
    perm = rng.permutation(pool)
    pm = np.full((n_req, n_pages), -1, dtype=np.int32)
    k = 0
    for r in range(n_req):
        for p in range(n_complete):
            if k < pool and rng.random() < 0.6:
                pm[r, p] = perm[k]
                k += 1
    return rng, pm, n_complete, pool


@pytest.mark.parametrize("seed", range(60))
def test_library_policy_matches_reference(seed):
    rng, pm, n_complete, pool = _scenario(seed)
    n_req = pm.shape[0]
    lib_pol = kvr.Residency(pm, n_complete, pool)
    ref = ResidencyPolicy(pm, n_complete, pool)
    handles = []
    try:
        for _ in range(40):
            op = int(rng.integers(0, 3))
            if op == 0:
                need = int(rng.integers(0, pool + 3))
                order = [int(x) for x in rng.permutation(n_req)[:int(rng.integers(0, n_req + 1))]]
                got = lib_pol.admit(need, order)
                want = ref.admit(need, order)
                assert got[0] == want[0] and got[1] == want[1]
                if got[0]:
                    handles.append((got[2], want[2]))
            elif op == 1 and handles:
                hl, hr = handles.pop(int(rng.integers(0, len(handles))))
                lib_pol.release(hl)
                ref.release(hr)
            else:
                bound = int(rng.integers(0, 8))
                assert lib_pol.refill(bound) == ref.refill(bound)
            assert lib_pol.counts() == ref.counts()
    finally:
        lib_pol.close()


def test_library_policy_rejects_bad_arguments():
    pm = np.array([[0, -1, 1], [-1, 2, -1]], dtype=np.int32)
    with pytest.raises(kvr.KvrError):
        kvr.Residency(np.array([[0, 0]], dtype=np.int32), 2, 4)  # one page mapped twice
    with pytest.raises(kvr.KvrError):
        kvr.Residency(np.array([[5]], dtype=np.int32), 1, 4)  # outside the pool
    pol = kvr.Residency(pm, 3, 4)
    try:
        with pytest.raises(kvr.KvrError):
            pol.admit(1, [0, 0])  # repeated request in the reclaim order
        with pytest.raises(kvr.KvrError):
            pol.admit(1, [2])  # request out of range
        with pytest.raises(kvr.KvrError):
            pol.release(7)  # unknown handle
        assert pol.counts() == (1, 3, 0)
        assert pol.admit(9, [0, 1]) == (False, [], -1)  # the admission waits
        assert pol.counts() == (1, 3, 0)
        ok, plan, h = pol.admit(3, [1, 0])
        assert ok and plan == [(1, 1), (0, 0), (0, 2)]
        assert pol.counts() == (1, 0, 3)
        pol.release(h)
        assert pol.refill(2) == [(0, 0, 0), (1, 1, 1)]  # the reclaimed pages come back
    finally:
        pol.close()
    lib = kvr.lib()
    assert lib.kvr_residency_admit(None, 0, 0, None, 0, None, None, None, None) == kvr.E_ARG
    assert lib.kvr_reclaim_pages(None, 0, None, None, None, None, None) == kvr.E_ARG
    assert lib.kvr_restore_pages(None, 0, None, None, None, None, None) == kvr.E_ARG
