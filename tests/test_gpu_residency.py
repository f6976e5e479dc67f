"""GPU parity of optional-pool residency: page reclaim (host backup, then
release) and restore (host rows into a physical page, then publish) against
the oracle, alone and between decode steps with an admission that forces a
deficit, its drain, and bounded round-robin refill.  The library's policy
decisions are compared with the reference policy's at every step."""
from __future__ import annotations

import numpy as np
import pytest

from oracle.residency import ResidencyPolicy
from oracle.runner import OracleRun
from synth import FULL, Inputs, tiny
from tests.test_gpu_parity import _compare_group, _compare_state

pytestmark = pytest.mark.gpu


def _gpu_run(inputs):
    from hierarchical_sparse_kv_resolve_amd.runner import GpuRun
    return GpuRun(inputs)


def _compare_pages(cfg, gpu, run, reqs):
    st = gpu.page_state()
    assert np.array_equal(st["page_map"][reqs], run.src.page_map), "page map"
    assert np.array_equal(st["host_valid"][reqs], run.src.host_valid), "host copies"
    mapped = sorted({int(ph) for ph in run.src.page_map.ravel() if ph >= 0})
    for l in range(cfg.payload_layers):
        assert np.array_equal(gpu.host[l][reqs], run.src.host[l]), f"host store, layer {l}"
        pool = gpu.pool[l].cpu().numpy()
        if reqs == list(range(cfg.n_req)):
            assert np.array_equal(pool, run.src.pool[l]), f"pool, layer {l}"
        else:
            assert np.array_equal(pool[mapped], run.src.pool[l][mapped]), f"pool, layer {l}"


@pytest.mark.parametrize("c", [2, 5])
def test_page_moves_alone(c):
    """Random reclaim and restore lists with repeats, pages that are not
    ready, trailing partial pages and bad entries."""
    from hierarchical_sparse_kv_resolve_amd import kvr
    cfg = tiny(c).with_(pool_spare=8)
    inputs = Inputs(cfg, max_new=4)
    gpu = _gpu_run(inputs)
    run = OracleRun(inputs)
    reqs = list(range(cfg.n_req))
    rng = np.random.default_rng(100 + c)
    try:
        for rnd in range(3):
            pm = run.src.page_map
            cand = [(r, p) for r in reqs for p in range(cfg.n_pages)]
            pick = [cand[i] for i in rng.choice(len(cand), size=min(len(cand), 12), replace=False)]
            pick += pick[:2]                                     # repeats
            pick += [(cfg.n_req, 0), (0, cfg.n_pages), (-1, 0)]  # bad entries
            order = rng.permutation(len(pick))
            req = np.array([pick[i][0] for i in order], dtype=np.int32)
            page = np.array([pick[i][1] for i in order], dtype=np.int32)
            fg, sg = gpu.reclaim_pages(list(zip(req.tolist(), page.tolist())))
            fo, so = run.src.reclaim_pages(req, page)
            assert np.array_equal(fg.cpu().numpy(), fo)
            assert np.array_equal(sg.cpu().numpy(), so)
            _compare_pages(cfg, gpu, run, reqs)
            # restore some not-ready complete pages into free physical pages,
            # with a repeated page, a repeated physical page and bad entries
            pm = run.src.page_map
            used = {int(x) for x in pm.ravel() if x >= 0}
            free = [ph for ph in range(cfg.pool_pages) if ph not in used]
            nr = [(r, p) for r in reqs for p in range(cfg.full_pages) if pm[r, p] < 0]
            nr = [nr[i] for i in rng.choice(len(nr), size=min(len(nr), len(free), 6), replace=False)]
            phys = [free[i] for i in rng.permutation(len(free))[:len(nr)]]
            placed = [(r, p, ph) for (r, p), ph in zip(nr, phys)]
            ready = [(r, p) for r in reqs for p in range(cfg.full_pages) if pm[r, p] >= 0][:1]
            extra = [(nr[0][0], nr[0][1], cfg.pool_pages - 1)] if nr else []
            if len(phys) > 1:
                extra.append((reqs[-1], cfg.full_pages, phys[1]))             # partial page
            extra += [(r, p, free[-1]) for r, p in ready]                     # already ready
            named = {(a, b) for a, b, _ in placed + extra}
            fresh = [(r, p) for r in reqs for p in range(cfg.full_pages)
                     if pm[r, p] < 0 and (r, p) not in named]
            extra += [(fresh[0][0], fresh[0][1], cfg.pool_pages)] if fresh else []  # E_RANGE
            extra += [(cfg.n_req, 0, 0)]                                          # bad request
            allp = placed + extra
            sg = gpu.restore_pages(allp)
            so = run.src.restore_pages([a for a, _, _ in allp], [b for _, b, _ in allp],
                                       [x for _, _, x in allp])
            assert np.array_equal(sg.cpu().numpy(), so)
            assert (so[:len(placed)] == kvr.OK).all() and (so[len(placed):] != kvr.OK).all()
            assert kvr.E_RANGE in so.tolist()
            _compare_pages(cfg, gpu, run, reqs)
            assert (run.src.check() == 0).all()
        # a corrupt map entry (an incomplete page marked ready) is refused
        part = cfg.full_pages
        assert cfg.H % cfg.P != 0
        gpu.page_map[0, part] = 0
        run.src.page_map[0, part] = 0
        fg, sg = gpu.reclaim_pages([(0, part)])
        fo, so = run.src.reclaim_pages([0], [part])
        assert fg.cpu().tolist() == fo.tolist() == [-1]
        assert sg.cpu().tolist() == so.tolist() == [kvr.E_STATE]
        gpu.page_map[0, part] = -1
        run.src.page_map[0, part] = -1
        _compare_pages(cfg, gpu, run, reqs)
    finally:
        gpu.close()


def _load_step(cfg, reqs, deficit, bound, admit_at, drain_at, prefetch_groups=0, sched=None,
               every_step=True):
    """every_step=False compares only after the last step, so that with the
    merged schedule each page move is issued while the previous step's last
    gather is still pending (the runner issues it first)."""
    from hierarchical_sparse_kv_resolve_amd import kvr
    inputs = Inputs(cfg, max_new=cfg.steps)
    gpu = _gpu_run(inputs)
    run = OracleRun(inputs, reqs=reqs)
    pol = kvr.Residency(inputs.page_map, cfg.full_pages, cfg.pool_pages)
    ref = ResidencyPolicy(inputs.page_map, cfg.full_pages, cfg.pool_pages)
    order = list(range(cfg.n_req))
    handles = None
    moved = 0
    try:
        for s in range(cfg.steps):
            if s == admit_at:
                got = pol.admit(cfg.pool_spare + deficit, order)
                want = ref.admit(cfg.pool_spare + deficit, order)
                assert got[:2] == want[:2] and got[0]
                handles = (got[2], want[2])
                fg, sg = gpu.reclaim_pages(got[1])
                fo, so = run.reclaim_pages(got[1])
                keep = [i for i, (r, _) in enumerate(got[1]) if r in reqs]
                assert np.array_equal(fg.cpu().numpy()[keep], fo)
                assert (sg.cpu().numpy() == 0).all() and (so == 0).all()
                moved += len(got[1])
            if s == drain_at:
                pol.release(handles[0])
                ref.release(handles[1])
            if s >= drain_at:
                placed = pol.refill(bound)
                assert placed == ref.refill(bound)
                sg = gpu.restore_pages(placed)
                so = run.restore_pages(placed)
                assert (sg.cpu().numpy() == 0).all() and (so == 0).all()
                moved += len(placed)
            assert pol.counts() == ref.counts()
            sels = [inputs.selections(s, g) for g in range(cfg.groups)]
            gpu.stage([s], sels={s: sels})
            o = run.step(s, sels=[x[reqs] for x in sels])
            gpu.step(s, prefetch_groups=prefetch_groups, **(sched or {}))
            if every_step or s == cfg.steps - 1:
                for g in range(cfg.groups):
                    _compare_group(cfg, gpu.group(g), o["groups"][g], reqs)
                    assert (o["groups"][g]["status"] == 0).all()
                _compare_state(gpu, run, reqs)
                _compare_pages(cfg, gpu, run, reqs)
            assert (run.src.check() == 0).all()
        assert moved > 0
    finally:
        pol.close()
        gpu.close()


@pytest.mark.parametrize("c,deficit,bound", [(2, 8, 2), (4, 12, 3), (5, 20, 4)])
def test_load_step_matches_oracle(c, deficit, bound):
    cfg = tiny(c).with_(pool_spare=5, steps=8)
    _load_step(cfg, list(range(cfg.n_req)), deficit, bound, admit_at=2, drain_at=4)


@pytest.mark.parametrize("every_step", [True, False])
@pytest.mark.parametrize("c,deficit,bound", [(2, 8, 2), (5, 20, 4)])
def test_load_step_merged_schedule(c, deficit, bound, every_step):
    """Page reclaim and refill between steps of the merged schedule, whose
    last gather of a step is still pending when the page moves are issued
    (compared after every step, or only after the last)."""
    cfg = tiny(c).with_(pool_spare=5, steps=8)
    _load_step(cfg, list(range(cfg.n_req)), deficit, bound, admit_at=2, drain_at=4,
               sched=dict(fused=True, merged=True), every_step=every_step)


def test_load_step_full_glm_sampled():
    """The GLM shape with a pool of spare pages: an admission takes four
    requests' optional pages, drains two steps later, and refill restores
    them 96 pages a step; the oracle follows requests 0, 3 and 6."""
    cfg = FULL[2].with_(pool_spare=64, steps=7)
    _load_step(cfg, [0, 3, 6], deficit=3 * cfg.ready_pages + 1, bound=96, admit_at=1,
               drain_at=3, prefetch_groups=2)
