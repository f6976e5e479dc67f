"""GPU parity of the speculative-state structures: the drafter visible-window
ring against its oracle (appends, rollbacks inside and outside the limit,
window gathers on request subsets), and verification staging reused across
payload layers while a slow consumer on another stream still reads them."""
from __future__ import annotations

import numpy as np
import pytest

from oracle.draft import DraftRing as RefRing
from oracle.runner import OracleRun
from synth import Inputs, payload_np, tiny

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,n_req,W,C,R", [(1, 5, 7, 11, 64), (2, 3, 16, 16, 576),
                                              (3, 8, 1, 4, 16), (4, 4, 12, 20, 656)])
def test_draft_ring_matches_oracle(seed, n_req, W, C, R):
    import torch
    from hierarchical_sparse_kv_resolve_amd import kvr
    rng = np.random.default_rng(seed)
    dev = "cuda"
    ring = torch.full((n_req, C, R), 0xAB, dtype=torch.uint8, device=dev)
    length = torch.full((n_req,), 7, dtype=torch.int32, device=dev)
    high = torch.full((n_req,), 7, dtype=torch.int32, device=dev)
    d = kvr.DraftRing(n_req, W, C, R, ring, length, high)
    d.reset()
    ref = RefRing(n_req, W, C, R)
    version = 0
    try:
        for _ in range(40):
            version += 1
            reqs = sorted(rng.choice(n_req, size=int(rng.integers(1, n_req + 1)), replace=False))
            req_d = torch.tensor(reqs, dtype=torch.int32, device=dev)
            n = len(reqs)
            op = rng.integers(0, 3)
            if op == 0:
                a = int(rng.integers(1, C + 1))
                rows = np.stack([payload_np(100 + version % 50, r,
                                            np.arange(int(ref.length[r]), int(ref.length[r]) + a),
                                            R, seed) for r in reqs])
                st = torch.full((n,), 9, dtype=torch.int32, device=dev)
                d.append(n, req_d, a, torch.from_numpy(rows).to(dev), st)
                ref.append(rows, reqs)
                assert (st.cpu().numpy() == 0).all()
            elif op == 1:
                keep = [int(rng.integers(0, int(ref.length[r]) + 2)) for r in reqs]
                st = torch.full((n,), 9, dtype=torch.int32, device=dev)
                d.rollback(n, req_d, torch.tensor(keep, dtype=torch.int32, device=dev), st)
                want = ref.rollback(keep, reqs)
                assert np.array_equal(st.cpu().numpy(), want)
            out = torch.full((n, W, R), 0xEE, dtype=torch.uint8, device=dev)
            vis = torch.zeros(n, dtype=torch.int32, device=dev)
            d.window(n, req_d, out, vis)
            want_out = np.full((n, W, R), 0xEE, dtype=np.uint8)
            want_vis = ref.window(want_out, reqs)
            assert np.array_equal(vis.cpu().numpy(), want_vis)
            assert np.array_equal(out.cpu().numpy(), want_out)
            assert np.array_equal(length.cpu().numpy(), ref.length.astype(np.int32))
            assert np.array_equal(high.cpu().numpy(), ref.high.astype(np.int32))
        # a request out of range is refused
        st = torch.zeros(1, dtype=torch.int32, device=dev)
        bad = torch.tensor([n_req], dtype=torch.int32, device=dev)
        d.window(1, bad, torch.zeros((1, W, R), dtype=torch.uint8, device=dev), None, st)
        assert st.cpu().tolist() == [kvr.E_ARG]
    finally:
        d.close()


def test_staging_reuse_waits_for_consumers():
    """Four payload layers gathered one at a time through two staging buffers;
    the consumer of each copies its buffer on another stream after a spin,
    so a buffer handed out again before its consumer finished would hold the
    next layer's rows when read."""
    import torch
    from hierarchical_sparse_kv_resolve_amd import kvr
    from hierarchical_sparse_kv_resolve_amd.runner import GpuRun
    cfg = tiny(4).with_(steps=3, payload_layers=4)
    assert cfg.q > 1
    inputs = Inputs(cfg, max_new=cfg.steps)
    gpu = GpuRun(inputs)
    run = OracleRun(inputs)
    pool = kvr.StagingPool(2)
    cons = torch.cuda.Stream()  # default priority
    main = torch.cuda.current_stream()
    stride = cfg.q * cfg.k
    staging = [torch.empty((cfg.n_req, stride, cfg.R), dtype=torch.uint8, device="cuda")
               for _ in range(2)]
    try:
        gpu.stage(range(cfg.steps))
        for s in range(cfg.steps):
            o = run.step(s)
            gpu.step(s, fused=True)
            results = [torch.full((cfg.n_req, stride, cfg.R), 0xEE, dtype=torch.uint8,
                                  device="cuda") for _ in range(cfg.payload_layers)]
            for l in range(cfg.payload_layers):
                idx = pool.acquire(main)
                gpu.ctx.gather_rows([l], cfg.n_req, None, gpu.loc[0], gpu.union_count, stride,
                                    [staging[idx]], stream=main)
                ready = torch.cuda.Event()
                ready.record(main)
                cons.wait_event(ready)
                with torch.cuda.stream(cons):
                    torch.cuda._sleep(2_000_000)  # a slow consumer
                    results[l].copy_(staging[idx])
                pool.release(idx, cons)
            torch.cuda.synchronize()
            rec = o["groups"][0]
            for l in range(cfg.payload_layers):
                got = results[l].cpu().numpy()
                for r in range(cfg.n_req):
                    u = rec["union_count"][r]
                    assert np.array_equal(got[r, :u], rec["out"][l][r, :u]), (s, l, r)
    finally:
        pool.close()
        gpu.close()
