"""Per-decode-step driver of the CPU reference over one synthetic workload.

TEST INFRASTRUCTURE ONLY.  A step is: append one decoded row per request,
then for every resolving layer in order: (verify block: take the union of
the queries' selections) -> resolve with host fill of payload layer 0 ->
(shared indices, distinct payloads: replay the fills into every other payload
layer) -> gather every payload layer with the one location vector.  Layers
that inherit a location vector from one physical source gather nothing more.

`reqs` restricts the reference to a subset of requests: requests never
interact, so the subset's results are exactly those of the full run.
"""
from __future__ import annotations

import numpy as np

from .oracle import OracleSource


class OracleRun:
    def __init__(self, inputs, reqs=None, pool=None, threads=None):
        cfg = inputs.cfg
        self.inputs, self.cfg = inputs, cfg
        self.reqs = list(range(cfg.n_req)) if reqs is None else [int(r) for r in reqs]
        n = len(self.reqs)
        nl = cfg.payload_layers
        if pool is None:
            pool = []
            for l in range(nl):
                p = np.empty((cfg.pool_pages, cfg.P, cfg.R), dtype=np.uint8)
                inputs.fill_pool(l, p)
                pool.append(p)
        tail, host = [], []
        for l in range(nl):
            t = np.empty((n, cfg.T, cfg.R), dtype=np.uint8)
            inputs.fill_tail(l, t, self.reqs)
            h = np.empty((n, inputs.host_rows, cfg.R), dtype=np.uint8)
            inputs.fill_host(l, h, self.reqs)
            tail.append(t)
            host.append(h)
        self.src = OracleSource(n_req=n, n_layers=nl, H=cfg.H, max_new=inputs.max_new, P=cfg.P,
                                T=cfg.T, B=cfg.B, R=cfg.R, page_map=inputs.page_map[self.reqs],
                                host_valid=inputs.host_valid[self.reqs], tail=tail, pool=pool,
                                host=host, threads=threads)

    def _local(self, r):
        return self.reqs.index(r) if r in self.reqs else -1

    def reclaim_pages(self, plan):
        """Apply a (request, page) list given in global request ids to the
        followed requests.  Returns (freed, status) of the applied entries."""
        keep = [(self._local(r), p) for r, p in plan if self._local(r) >= 0]
        return self.src.reclaim_pages([r for r, _ in keep], [p for _, p in keep])

    def restore_pages(self, placed):
        """Apply a (request, page, physical page) list given in global request
        ids to the followed requests.  Returns the status of applied entries."""
        keep = [(self._local(r), p, ph) for r, p, ph in placed if self._local(r) >= 0]
        return self.src.restore_pages([r for r, _, _ in keep], [p for _, p, _ in keep],
                                      [ph for _, _, ph in keep])

    def step(self, s: int, sels=None) -> dict:
        """Run decode step s.  `sels` may supply the per-group selections
        (int32 [n][q][k]); otherwise they come from the generator."""
        cfg, src = self.cfg, self.src
        out = {"append_status": src.append(self.inputs.new_rows(s, self.reqs)), "groups": []}
        for g in range(cfg.groups):
            sel = self.inputs.selections(s, g, self.reqs) if sels is None else sels[g]
            rec = {"sel": sel}
            if cfg.q > 1:
                union, ucount, mp = src.dedup(sel)
                rec.update(union=union, union_count=ucount, map=mp)
                loc, fills, fc, st = src.resolve(union, count=ucount, fill_layer=0)
                count = ucount
            else:
                loc, fills, fc, st = src.resolve(sel[:, 0, :], fill_layer=0)
                count = None
            rec.update(loc=loc, fills=fills, fill_count=fc, status=st, count=count)
            if cfg.reuse == "distinct":
                for l in range(1, cfg.payload_layers):
                    src.replay(l, fills, fc)
                rec["out"] = [src.gather(l, loc, count)[0] for l in range(cfg.payload_layers)]
            else:
                rec["out"] = [src.gather(0, loc, count)[0]]
            out["groups"].append(rec)
        return out
