"""Per-decode-step driver of the GPU resolver over one workload.

Owns the device buffers (torch allocates them; pinned host stores come from
kvr_host_alloc), binds them to a libkvr context and issues, per decode step,
stream-ordered calls with no host synchronisation.  The one-stream schedule:

  append one decoded row per request (all payload layers; by default inside
  the first resolve launch: append_resolve_rows)
  for each resolving layer, in order:
      [verify block]  dedup_verify_selections -> union
      resolve_rows    (tail / ready page / hot scan / LRU victims; host refill
                       of payload layer 0)
      shared indices, distinct payloads: reuse_locations(DISTINCT_PAYLOAD)
                       replays the fills into every other payload layer, then
                       one gather_rows over all payload layers
      one physical source: gather_rows of the source, then
                       reuse_locations(SHARED_SOURCE) for each Reuse layer
                       (an alias: no bytes move)

The other schedules (GpuRun.step) reorder the fills and gathers of the same
calls: prefetch issues the host fills of layer groups on a side stream ahead
of their gathers; fused fills from host and gathers in one launch
(fused_gather_rows); pipelined runs each resolve on the current stream while
the previous fused launch gathers on a side stream; merged (the default of
bench.py) issues each resolve in one launch with the gather of the resolve
before it (gather_resolve_rows) and leaves the last gather to finish().
Every schedule gives the same results.

`inputs` supplies shapes and seeded contents (cfg, page_map, host_valid,
fill_tail/fill_pool/fill_host, new_rows, selections).
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import kvr


def layer_groups(n_layers: int, prefetch_groups) -> list:
    """Payload layers split into consecutive groups: G equal groups for an
    int G, or the given group sizes."""
    if isinstance(prefetch_groups, int):
        return np.array_split(np.arange(n_layers), min(prefetch_groups, n_layers))
    sizes = [int(x) for x in prefetch_groups]
    if any(x <= 0 for x in sizes) or sum(sizes) != n_layers:
        raise ValueError(f"group sizes {sizes} do not split {n_layers} layers")
    return np.split(np.arange(n_layers), np.cumsum(sizes)[:-1])


class GpuRun:
    def __init__(self, inputs, pool_host=None, device: str = "cuda", fuse_append: bool = True,
                 step_buffers: int = 0):
        """fuse_append: the step's append runs inside its first resolve launch
        (kvr_append_resolve_rows) instead of as a launch of its own.
        step_buffers: sets of per-step output buffers that alternate by step
        (0: two when a step has one resolving layer, else one); more sets
        let the pipelined schedule's resolves run further ahead."""
        import torch
        self.torch = torch
        self.fuse_append = fuse_append
        cfg = inputs.cfg
        self.cfg, self.inputs = cfg, inputs
        dev = torch.device(device)
        self.dev = dev
        n, nl = cfg.n_req, cfg.payload_layers
        self.n, self.nl = n, nl
        self.ctx = kvr.Context(n_req=n, n_layers=nl, history_rows=cfg.H,
                               max_new_rows=inputs.max_new, page_rows=cfg.P, tail_rows=cfg.T,
                               hot_slots=cfg.B, row_bytes=cfg.R, sel_cap=cfg.sel_cap,
                               pool_pages=cfg.pool_pages)
        i32 = torch.int32
        self.L = torch.empty(n, dtype=i32, device=dev)
        self.page_map = torch.from_numpy(np.ascontiguousarray(inputs.page_map)).to(dev)
        self.host_valid = torch.from_numpy(np.ascontiguousarray(inputs.host_valid)).to(dev)
        self.tag = torch.empty((n, cfg.B), dtype=i32, device=dev)
        self.stamp = torch.empty((n, cfg.B), dtype=i32, device=dev)   # uint32 bits
        self.clock = torch.empty(n, dtype=i32, device=dev)            # uint32 bits
        self.ctx.bind_metadata(self.L, self.page_map, self.host_valid, self.tag, self.stamp,
                               self.clock)
        self.tail, self.pool, self.hot, self.host_ptr, self.host = [], [], [], [], []
        host_bytes = n * inputs.host_rows * cfg.R
        for l in range(nl):
            t = np.empty((n, cfg.T, cfg.R), dtype=np.uint8)
            inputs.fill_tail(l, t)
            self.tail.append(torch.from_numpy(t).to(dev))
            if pool_host is not None:
                p = pool_host[l]
            else:
                p = np.empty((cfg.pool_pages, cfg.P, cfg.R), dtype=np.uint8)
                inputs.fill_pool(l, p)
            self.pool.append(torch.from_numpy(p).to(dev))
            self.hot.append(torch.full((n, cfg.B, cfg.R), 0xCD, dtype=torch.uint8, device=dev))
            ptr = kvr.host_alloc(host_bytes)
            self.host_ptr.append(ptr)
            view = np.ctypeslib.as_array((ctypes.c_uint8 * host_bytes).from_address(ptr))
            view = view.reshape(n, inputs.host_rows, cfg.R)
            inputs.fill_host(l, view)
            self.host.append(view)
            self.ctx.bind_layer(l, self.tail[l] if cfg.T else None,
                                self.pool[l] if cfg.pool_pages else None, self.hot[l], ptr)
        self.ctx.init_state()
        G, cap = cfg.groups, cfg.sel_cap
        # The per-call outputs of a step (locations, fills, status, verify
        # union, appended positions).  With one resolving layer per step two
        # sets alternate by step parity, so that in the pipelined schedule
        # the next step's resolve does not overwrite what this step's gather
        # still reads; with several resolving layers each layer's set is
        # rewritten only a whole step later.  The attributes below always
        # name the set of the step issued last.
        self._nbuf = step_buffers if step_buffers > 0 else (2 if G == 1 else 1)
        self._sets = []
        for _ in range(self._nbuf):
            bs = {"loc": [torch.empty((n, cap), dtype=i32, device=dev) for _ in range(G)],
                  "fills": [torch.empty((n, cfg.B, 2), dtype=i32, device=dev) for _ in range(G)],
                  "fill_count": [torch.empty(n, dtype=i32, device=dev) for _ in range(G)],
                  "status": [torch.empty(n, dtype=i32, device=dev) for _ in range(G)],
                  "append_pos": torch.empty(n, dtype=i32, device=dev)}
            if cfg.q > 1:
                bs.update(union=torch.empty((n, cfg.q * cfg.k), dtype=i32, device=dev),
                          union_count=torch.empty(n, dtype=i32, device=dev),
                          map=torch.empty((n, cfg.q, cfg.k), dtype=i32, device=dev))
            self._sets.append(bs)
        self._use_set(0)
        self.append_status = torch.empty(n, dtype=i32, device=dev)
        self.gather_status = torch.zeros(n, dtype=i32, device=dev)
        self.stats = torch.zeros(len(kvr.STATS_FIELDS), dtype=torch.int64, device=dev)
        n_out = nl if cfg.reuse == "distinct" else 1
        self.outs = [[torch.full((n, cap, cfg.R), 0xEE, dtype=torch.uint8, device=dev)
                      for _ in range(n_out)] for _ in range(G)]
        self.sel_dev, self.rows_dev = {}, {}
        # Every stream a schedule may use exists before any step is issued or
        # captured, and the events a step records stay referenced until the
        # step (or a whole capture) is done, so no stream or event is created
        # or destroyed while a capture is open.
        self._side_streams = {k: torch.cuda.Stream() for k in (1, 2)}  # default priority
        self._events = []
        # pipelined schedule: the side-stream event after the last gather
        # that read each (buffer set, group), and after the last side launch
        self._gather_done = {}
        self._side_last = None
        # merged schedule: the gather of the last resolve, not yet issued
        self._pending = None

    def _use_set(self, b: int):
        bs = self._sets[b]
        self.loc, self.fills = bs["loc"], bs["fills"]
        self.fill_count, self.status = bs["fill_count"], bs["status"]
        self.append_pos = bs["append_pos"]
        if self.cfg.q > 1:
            self.union, self.union_count, self.map = bs["union"], bs["union_count"], bs["map"]

    def finish(self, stream=None):
        """Complete the steps issued so far on `stream` (default: the current
        one): issue the merged schedule's last gather, and wait for the
        pipelined schedule's side-stream work.  No host wait."""
        st = stream or self.torch.cuda.current_stream()
        if self._pending is not None:
            self.ctx.gather_resolve_rows(gather=self._pending, resolve=None, stream=st)
            self._pending = None
        if self._side_last is not None:
            st.wait_event(self._side_last)

    def close(self):
        self.torch.cuda.synchronize()
        self.ctx.close()
        for p in self.host_ptr:
            kvr.host_free(p)
        self.host_ptr = []

    # ------------------------------------------------------------------
    def stage(self, steps, sels=None):
        """Copy the selections and new rows of `steps` to the device (before timing).
        sels: optional {step: [per-group int32 [n][q][k]]}."""
        torch = self.torch
        for s in steps:
            gs = sels[s] if sels is not None and s in sels else [
                self.inputs.selections(s, g) for g in range(self.cfg.groups)]
            self.sel_dev[s] = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(self.dev)
                               for x in gs]
            self.rows_dev[s] = torch.from_numpy(self.inputs.new_rows(s)).to(self.dev)

    def step(self, s: int, prefetch_groups=0, serialize: bool = False, fused: bool = False,
             pipelined: bool = False, merged: bool = False):
        """Enqueue decode step s (staged beforehand) on the current stream.  No
        host synchronisation.

        pipelined=True (with fused=True, not serialized): the fused schedule
        with every fused launch on a side stream and every resolve on the
        current stream, and nothing joining the two at the end of a step, so
        that the next step's resolve runs while this step's last fused launch
        gathers.  The step's append is deferred (append_resolve_rows_deferred
        writes the host copy and the length) and completed by the step's
        first fused launch (fused_gather_append_rows), because the tail slot
        it overwrites may still be read by the previous step's gather.  A
        resolve waits only for the gather that last read its output buffers.
        Call finish() before work on the current stream that needs this
        step's gathered rows or hot payload (capture() and the read-back
        helpers do).

        merged=True (with fused=True, not serialized): the same overlap on
        one stream with no wait between queues: each resolve is issued in
        one launch with the gather of the resolve before it
        (gather_resolve_rows), and the step's last gather waits for the next
        step's first resolve, or for finish().

        prefetch_groups = 0: resolve fills payload layer 0 from host, one
        replay call fills the other layers, one gather call covers them all.
        prefetch_groups = G > 0: with shared indices and distinct payloads the
        host fills of all layers are issued on a side stream in G groups of
        layers, and each group's gather starts on the current stream as soon
        as that group's fills are in, so host-link traffic of later groups
        overlaps the HBM traffic of earlier gathers.  A sequence of group
        sizes (summing to the layer count) sets the groups explicitly:
        shrinking groups leave only a small last gather after the last fill.  With one physical source
        and several resolving layers, each layer's fill and gather run on the
        side stream while the next layer resolves.

        fused=True (prefetch_groups is then ignored): the host fill and the
        gather of fresh rows are one pass while every other row is gathered
        beside it, as one launch (fused_gather_rows): on the current stream
        with distinct payloads; with one physical source and several
        resolving layers, on a side stream while the current stream resolves
        the next layer.

        serialize=True issues the same work but lets no two launches
        overlap, so launch timing (Context.timing_begin) sees each kernel
        running alone; each fused launch is then issued as its two halves
        (fill_gather_rows, then gather_resident_rows), so that each half is
        timed alone (for one physical source on two side streams that wait
        on each other's events)."""
        torch = self.torch
        cfg, ctx, n = self.cfg, self.ctx, self.n
        if not getattr(self, "_capturing", False):
            # the previous step's events (those later steps of the pipelined
            # schedule wait on stay referenced by _gather_done / _side_last)
            self._events = []
        self._use_set(s % self._nbuf)
        if pipelined or merged:
            if not fused or serialize or not self.fuse_append or (pipelined and merged):
                raise ValueError("the pipelined and merged schedules are the fused one, not "
                                 "serialized, with the append inside the first resolve")
            if merged:
                self._step_merged(s)
            else:
                self._step_pipelined(s)
            return
        self.finish()  # other schedules start from a joined side stream
        main = torch.cuda.current_stream()
        last_filled = last_resident = None
        if not self.fuse_append:
            ctx.append_rows(n, None, self.rows_dev[s], self.append_status, stream=main)
        for g in range(cfg.groups):
            sel = self.sel_dev[s][g]
            k = sel.shape[-1]
            if cfg.q > 1:
                ctx.dedup_verify_selections(n, cfg.q, k, sel, self.union, self.union_count,
                                            self.map, stream=main)
                src, count, stride = self.union, self.union_count, cfg.q * k
            else:
                src, count, stride = sel, None, k
            loc, fills, fc = self.loc[g], self.fills[g], self.fill_count[g]
            # the host fills are issued apart from the resolve (prefetch
            # groups, or the fused fill-and-gather), not by the resolve call
            fills_apart = bool(prefetch_groups) or fused
            fill_layer = -1 if fills_apart else 0
            if self.fuse_append and g == 0:
                ctx.append_resolve_rows(n, None, self.rows_dev[s], self.append_status, src, count,
                                        stride, loc, fills, fc, fill_layer, self.status[g],
                                        self.stats, stream=main)
            else:
                ctx.resolve_rows(n, None, src, count, stride, loc, fills, fc, fill_layer,
                                 self.status[g], self.stats, stream=main)
            if fused and cfg.reuse == "distinct" and not serialize:
                ctx.fused_gather_rows(list(range(self.nl)), n, None, loc, src, count, stride,
                                      self.outs[g], self.gather_status, stream=main)
            elif fused and not serialize:
                # One physical source: each layer's fused launch runs on the
                # side stream while the main stream resolves the next layer
                # (resolve touches metadata only); on one stream the next
                # layer's fill comes after this layer's resident gather (its
                # victims may be slots that gather reads) and its resident
                # gather after this fill (its hits may be slots the fill wrote).
                resolved = self._event()
                resolved.record(main)
                side = self._side()
                side.wait_event(resolved)
                ctx.fused_gather_rows([0], n, None, loc, src, count, stride, self.outs[g][:1],
                                      self.gather_status, stream=side)
                for _ in range(1, cfg.layers_per_group):
                    ctx.reuse_locations(kvr.REUSE_SHARED_SOURCE, None, n, None, loc, None, count,
                                        stride, stream=main)
                if g == cfg.groups - 1:
                    done = self._event()
                    done.record(side)
                    main.wait_event(done)
            elif fused:
                resolved = self._event()
                resolved.record(main)
                side = self._side()
                side.wait_event(resolved)
                layers = list(range(self.nl)) if cfg.reuse == "distinct" else [0]
                outs = self.outs[g] if cfg.reuse == "distinct" else self.outs[g][:1]
                if cfg.reuse != "distinct" and last_resident is not None:
                    side.wait_event(last_resident)
                ctx.fill_gather_rows(layers, n, None, loc, src, count, stride, outs,
                                     self.gather_status, stream=side)
                filled = self._event()
                filled.record(side)
                res = main if cfg.reuse == "distinct" else self._side(2)
                res.wait_event(resolved)
                if serialize:
                    res.wait_event(filled)
                elif last_filled is not None:
                    res.wait_event(last_filled)
                ctx.gather_resident_rows(layers, n, None, loc, count, stride, outs,
                                         self.gather_status, stream=res)
                resident = self._event()
                resident.record(res)
                last_filled, last_resident = filled, resident
                for _ in range(1, cfg.layers_per_group):
                    ctx.reuse_locations(kvr.REUSE_SHARED_SOURCE, None, n, None, loc, None, count,
                                        stride, stream=main)
                if g == cfg.groups - 1 or serialize:
                    main.wait_event(filled)
                    main.wait_event(resident)
            elif cfg.reuse != "distinct" and fills_apart:
                # One physical source: this layer's fill and gather run on the
                # side stream while the main stream resolves the next layer
                # (resolve touches metadata only).  The side stream keeps the
                # next fill behind this gather: its victims may be slots this
                # gather still reads.
                resolved = self._event()
                resolved.record(main)
                side = self._side()
                side.wait_event(resolved)
                ctx.reuse_locations(kvr.REUSE_DISTINCT_PAYLOAD, [0], n, None, loc, None,
                                    count, stride, fills, fc, stream=side)
                ctx.gather_rows([0], n, None, loc, count, stride, self.outs[g][:1],
                                self.gather_status, stream=side)
                for _ in range(1, cfg.layers_per_group):
                    ctx.reuse_locations(kvr.REUSE_SHARED_SOURCE, None, n, None, loc, None, count,
                                        stride, stream=side)
                if g == cfg.groups - 1 or serialize:
                    done = self._event()
                    done.record(side)
                    main.wait_event(done)
            elif cfg.reuse != "distinct":
                if fill_layer < 0:
                    ctx.reuse_locations(kvr.REUSE_DISTINCT_PAYLOAD, [0], n, None, loc, None,
                                        count, stride, fills, fc, stream=main)
                ctx.gather_rows([0], n, None, loc, count, stride, self.outs[g][:1],
                                self.gather_status, stream=main)
                for _ in range(1, cfg.layers_per_group):
                    ctx.reuse_locations(kvr.REUSE_SHARED_SOURCE, None, n, None, loc, None, count,
                                        stride, stream=main)
            elif not fills_apart:
                layers = list(range(1 if fill_layer == 0 else 0, self.nl))
                if layers:
                    ctx.reuse_locations(kvr.REUSE_DISTINCT_PAYLOAD, layers, n, None, loc,
                                        None, count, stride, fills, fc, stream=main)
                ctx.gather_rows(list(range(self.nl)), n, None, loc, count, stride,
                                self.outs[g], self.gather_status, stream=main)
            else:
                groups = layer_groups(self.nl, prefetch_groups)
                resolved = self._event()
                resolved.record(main)
                side = self._side()
                side.wait_event(resolved)
                ready = []
                for grp in groups:
                    ctx.reuse_locations(kvr.REUSE_DISTINCT_PAYLOAD, grp.tolist(), n, None,
                                        loc, None, count, stride, fills, fc, stream=side)
                    ev = self._event()
                    ev.record(side)
                    ready.append(ev)
                if serialize:
                    ready = [ready[-1]] * len(ready)  # every fill before the first gather
                for grp, ev in zip(groups, ready):
                    main.wait_event(ev)
                    ctx.gather_rows(grp.tolist(), n, None, loc, count, stride,
                                    [self.outs[g][l] for l in grp], self.gather_status,
                                    stream=main)

    def _step_merged(self, s: int):
        torch = self.torch
        cfg, ctx, n = self.cfg, self.ctx, self.n
        main = torch.cuda.current_stream()
        distinct = cfg.reuse == "distinct"
        layers = list(range(self.nl)) if distinct else [0]
        for g in range(cfg.groups):
            sel = self.sel_dev[s][g]
            k = sel.shape[-1]
            if cfg.q > 1:
                ctx.dedup_verify_selections(n, cfg.q, k, sel, self.union, self.union_count,
                                            self.map, stream=main)
                src, count, stride = self.union, self.union_count, cfg.q * k
            else:
                src, count, stride = sel, None, k
            loc, fills, fc = self.loc[g], self.fills[g], self.fill_count[g]
            res = dict(n=n, sel=src, sel_count=count, stride=stride, loc=loc, fills=fills,
                       fill_count=fc, status=self.status[g], stats=self.stats)
            if g == 0:
                res.update(new_rows=self.rows_dev[s], append_status=self.append_status,
                           append_pos=self.append_pos)
            ctx.gather_resolve_rows(gather=self._pending, resolve=res, stream=main)
            gat = dict(layers=layers, n=n, loc=loc, sel=src, count=count, stride=stride,
                       outs=self.outs[g] if distinct else self.outs[g][:1],
                       status=self.gather_status)
            if g == 0:
                gat.update(new_rows=self.rows_dev[s], append_pos=self.append_pos)
            self._pending = gat
            if not distinct:
                for _ in range(1, cfg.layers_per_group):
                    ctx.reuse_locations(kvr.REUSE_SHARED_SOURCE, None, n, None, loc, None, count,
                                        stride, stream=main)

    def _step_pipelined(self, s: int):
        torch = self.torch
        cfg, ctx, n = self.cfg, self.ctx, self.n
        main, side = torch.cuda.current_stream(), self._side()
        b = s % self._nbuf
        distinct = cfg.reuse == "distinct"
        layers = list(range(self.nl)) if distinct else [0]
        for g in range(cfg.groups):
            sel = self.sel_dev[s][g]
            k = sel.shape[-1]
            free = self._gather_done.get((b, g))
            if free is not None:
                main.wait_event(free)  # the gather that last read this set's buffers
            if cfg.q > 1:
                ctx.dedup_verify_selections(n, cfg.q, k, sel, self.union, self.union_count,
                                            self.map, stream=main)
                src, count, stride = self.union, self.union_count, cfg.q * k
            else:
                src, count, stride = sel, None, k
            loc, fills, fc = self.loc[g], self.fills[g], self.fill_count[g]
            if g == 0:
                ctx.append_resolve_rows_deferred(n, None, self.rows_dev[s], self.append_status,
                                                 self.append_pos, src, count, stride, loc, fills,
                                                 fc, -1, self.status[g], self.stats, stream=main)
            else:
                ctx.resolve_rows(n, None, src, count, stride, loc, fills, fc, -1, self.status[g],
                                 self.stats, stream=main)
            resolved = self._event()
            resolved.record(main)
            side.wait_event(resolved)
            outs = self.outs[g] if distinct else self.outs[g][:1]
            if g == 0:
                ctx.fused_gather_append_rows(layers, n, None, loc, src, count, stride, outs,
                                             self.rows_dev[s], self.append_pos,
                                             self.gather_status, stream=side)
            else:
                ctx.fused_gather_rows(layers, n, None, loc, src, count, stride, outs,
                                      self.gather_status, stream=side)
            done = self._event()
            done.record(side)
            self._gather_done[(b, g)] = done
            self._side_last = done
            if not distinct:
                for _ in range(1, cfg.layers_per_group):
                    ctx.reuse_locations(kvr.REUSE_SHARED_SOURCE, None, n, None, loc, None, count,
                                        stride, stream=main)

    # ------------------------------------------------------------------ residency
    def reclaim_pages(self, plan, stream=None):
        """Enqueue the release of the (request, page) list `plan` (host backup
        of pages without one first).  Returns device tensors (freed physical
        page or -1, status) per entry."""
        torch = self.torch
        self.finish(stream)  # a pending gather may still read the pages
        n = len(plan)
        req = torch.tensor([r for r, _ in plan] or [0], dtype=torch.int32, device=self.dev)
        page = torch.tensor([p for _, p in plan] or [0], dtype=torch.int32, device=self.dev)
        freed = torch.full((max(1, n),), -1, dtype=torch.int32, device=self.dev)
        status = torch.zeros(max(1, n), dtype=torch.int32, device=self.dev)
        self.ctx.reclaim_pages(n, req, page, freed, status, stream=stream)
        return freed[:n], status[:n]

    def restore_pages(self, placed, stream=None):
        """Enqueue making the (request, page, physical page) list ready.
        Returns the device status tensor per entry."""
        torch = self.torch
        self.finish(stream)  # a pending gather may still read the pool
        n = len(placed)
        cols = list(zip(*placed)) if placed else [[0], [0], [0]]
        req, page, phys = (torch.tensor(list(c), dtype=torch.int32, device=self.dev) for c in cols)
        status = torch.zeros(max(1, n), dtype=torch.int32, device=self.dev)
        self.ctx.restore_pages(n, req, page, phys, status, stream=stream)
        return status[:n]

    def page_state(self) -> dict:
        self.torch.cuda.synchronize()
        return {"page_map": self.page_map.cpu().numpy(), "host_valid": self.host_valid.cpu().numpy()}

    def snapshot(self) -> dict:
        """Device copies of the mutable state (metadata, hot caches, tails)."""
        self.finish()
        return {"L": self.L.clone(), "tag": self.tag.clone(), "stamp": self.stamp.clone(),
                "clock": self.clock.clone(), "hot": [h.clone() for h in self.hot],
                "tail": [t.clone() for t in self.tail], "stats": self.stats.clone()}

    def restore(self, snap: dict) -> None:
        self.finish()
        for name in ("L", "tag", "stamp", "clock", "stats"):
            getattr(self, name).copy_(snap[name])
        for dst, src in zip(self.hot, snap["hot"]):
            dst.copy_(src)
        for dst, src in zip(self.tail, snap["tail"]):
            dst.copy_(src)

    def capture(self, steps, prefetch_groups=0, fused: bool = False, pipelined: bool = False,
                merged: bool = False):
        """Capture the launches of `steps` into one HIP graph (nothing runs
        until it is replayed).  Each replay runs those decode steps again from
        whatever state the buffers hold."""
        torch = self.torch
        if fused and self.cfg.reuse != "distinct":
            # Capturing this schedule in an earlier form (the fill and the
            # resident gathers as two launches on two side streams that waited
            # on each other's events across resolving layers) ended in a host
            # crash inside the graph runtime's capture end.  No cause was
            # found, so this schedule is not captured in any form; eager runs
            # are unaffected.
            raise NotImplementedError("graph capture of the fused schedule for one physical "
                                      "source with several resolving layers is disabled")
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()  # default priority
        self.finish()
        cap.wait_stream(torch.cuda.current_stream())
        # no wait inside the capture on an event recorded before it
        self._gather_done, self._side_last = {}, None
        self._capturing = True
        try:
            with torch.cuda.stream(cap):
                with torch.cuda.graph(graph, stream=cap):
                    for s in steps:
                        self.step(s, prefetch_groups=prefetch_groups, fused=fused,
                                  pipelined=pipelined, merged=merged)
                    # the last gather, and the side stream joins, before the capture ends
                    self.finish(cap)
        finally:
            self._capturing = False
            self._events = []
            self._gather_done, self._side_last, self._pending = {}, None, None
        torch.cuda.current_stream().wait_stream(cap)
        return graph

    def _side(self, k: int = 1):
        return self._side_streams[k]

    def _event(self):
        """A new event, kept referenced until the step or capture ends."""
        ev = self.torch.cuda.Event()
        self._events.append(ev)
        return ev

    # ------------------------------------------------------------------ read-back (syncs)
    def state(self) -> dict:
        self.finish()
        self.torch.cuda.synchronize()
        return {"L": self.L.cpu().numpy(), "tag": self.tag.cpu().numpy(),
                "stamp": self.stamp.cpu().numpy().view(np.uint32),
                "clock": self.clock.cpu().numpy().view(np.uint32)}

    def group(self, g: int, with_out: bool = True) -> dict:
        self.finish()
        self.torch.cuda.synchronize()
        rec = {"loc": self.loc[g].cpu().numpy().view(np.uint32),
               "fills": self.fills[g].cpu().numpy(),
               "fill_count": self.fill_count[g].cpu().numpy(),
               "status": self.status[g].cpu().numpy()}
        if self.cfg.q > 1:
            rec.update(union=self.union.cpu().numpy(), union_count=self.union_count.cpu().numpy(),
                       map=self.map.cpu().numpy())
        if with_out:
            rec["out"] = [o.cpu().numpy() for o in self.outs[g]]
        return rec

    def stats_dict(self) -> dict:
        vals = self.stats.cpu().numpy().astype(np.uint64)
        return dict(zip(kvr.STATS_FIELDS, (int(v) for v in vals)))
