"""Benchmark of the per-decode-step sparse KV row resolver on one MI355X.

A step is one pass of the whole resolver path over one batch: append one
decoded row per request, then per resolving layer: (verify-block dedup),
resolve (tail / ready page / hot-cache scan / LRU victims), host refill of
the missing rows, per-layer replays for layers that share indices with
distinct payloads, and the multi-layer gather into contiguous buffers.
Inputs (selections, new rows, payload) are seeded synthetic data, staged
in HBM and pinned host memory before the timed region.

Prints one JSON line.  `value` is selected rows resolved+gathered per
second: (request, payload layer, selected row) entries written by the
gather; rows of layers that only inherit a location vector are not counted.

  python bench.py [--steps K] [--warmup W] [--workload c5] [--no-cpu-baseline]

The default workload is the largest: DeepSeek-style long context (64
requests of 524288-row histories, 4 resolving + 8 Reuse layers, 22 GB pinned
host store).
"""
from __future__ import annotations

import argparse
import contextlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# MI355X's host interface is PCIe 5.0 x16: 128 GB/s both ways, 64 GB/s in
# one direction (host to device is the direction the fills use)
HOST_LINK_PEAK_GBS = 64.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=28)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="c5", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--cpu-requests", type=int, default=16,
                    help="requests the CPU baseline runs (a bounded sample of the workload's; "
                         "requests never interact, so rows/s is per request processed)")
    ap.add_argument("--no-graph", action="store_true",
                    help="issue the timed steps eagerly instead of replaying one HIP graph")
    ap.add_argument("--prefetch-groups", default="2",
                    help="layer groups whose host fills overlap earlier gathers: a count "
                         "(equal groups, 0 = off) or comma-separated group sizes")
    ap.add_argument("--schedule", default="auto",
                    choices=["auto", "prefetch", "fused", "pipelined", "merged"],
                    help="fused: host fills and the gather of the rows they bring in as one "
                         "pass beside the gather of all other rows; pipelined: the fused "
                         "launches on a side stream so that each resolve (the next step's "
                         "included) runs beside the previous gathers; merged: the same overlap "
                         "in one launch per resolve (gather of the previous resolve beside "
                         "it) on one stream; prefetch: fills in layer groups ahead of "
                         "per-group gathers; auto: merged")
    ap.add_argument("--step-buffers", type=int, default=0,
                    help="sets of per-step output buffers (0: the runner's default)")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed runs of the K steps from the same state (median reported)")
    ap.add_argument("--hot-slots", type=int, default=0,
                    help="hot-cache budget B per request (default: the workload's)")
    ap.add_argument("--scenario", default="", choices=["", "load_step"],
                    help="load_step: optional-pool residency under an admission that "
                         "forces reclamation, then its drain and bounded refill")
    ap.add_argument("--refill-bound", type=int, default=16,
                    help="load_step: optional pages refilled per decode step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain device copies of known size (for scaling the "
                         "HBM byte counters) and exit")
    return ap.parse_args()


def launch_means_ms(records):
    """{kernel name: [durations in ms]} from (name, ms) launch records."""
    out = {}
    for name, ms in records:
        out.setdefault(name, []).append(ms)
    return out


def rows_per_group(inputs, steps):
    """Per (step, group): rows resolved by the call (union size for verify)."""
    cfg = inputs.cfg
    out = {}
    for s in steps:
        for g in range(cfg.groups):
            sel = inputs.selections(s, g)
            if cfg.q > 1:
                out[(s, g)] = sum(len(np.unique(sel[r])) for r in range(cfg.n_req))
            else:
                out[(s, g)] = sel.shape[0] * sel.shape[2]
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def auto_schedule(cfg) -> str:
    """The default schedule: merged (each resolve in one launch with the
    gather of the resolve before it), which measured fastest or even on
    every workload: single request 11.0 us per step (fused 16.6), GLM
    221 us (fused 241), memory pressure 2.247 ms (prefetch 2.311), verify
    0.704 ms (pipelined 0.704, fused 0.733), long context 2.886 ms (fused
    2.977)."""
    return "merged"


def schedule_kwargs(schedule: str) -> dict:
    """GpuRun.step flags of a schedule name (prefetch groups aside)."""
    return dict(fused=schedule in ("fused", "pipelined", "merged"),
                pipelined=schedule == "pipelined", merged=schedule == "merged")


def cpu_baseline(cfg, total_steps, budget_s, min_s=10.0, threads=None, n_reqs=None):
    """The oracle as it stands, on this host's cores (or `threads` of them),
    over the same decode steps from a fresh state, for the first `n_reqs`
    requests (all by default); the pass is repeated (state restored) until at
    least `min_s` seconds of work, and stops early at `budget_s`."""
    from oracle.runner import OracleRun
    from synth import Inputs
    inputs = Inputs(cfg, max_new=total_steps)
    n = cfg.n_req if not n_reqs else min(n_reqs, cfg.n_req)
    reqs = list(range(n))
    run = OracleRun(inputs, reqs=reqs, threads=threads)
    src = run.src
    snap = src.snapshot()
    sels = {s: [inputs.selections(s, g, reqs) for g in range(cfg.groups)]
            for s in range(total_steps)}
    n_out = cfg.payload_layers if cfg.reuse == "distinct" else 1
    rows = 0
    spent = 0.0
    passes = 0
    steps_done = 0
    while spent < min_s and spent < budget_s:
        for name in ("L", "tag", "stamp", "clock"):
            np.copyto(getattr(src, name), snap[name])
        for l in range(src.n_layers):
            np.copyto(src.hot[l], snap["hot"][l])
            np.copyto(src.tail[l], snap["tail"][l])
        t0 = time.perf_counter()
        for s in range(total_steps):
            res = run.step(s, sels=sels[s])
            for rec in res["groups"]:
                cnt = rec["count"]
                per = int(cnt.sum()) if cnt is not None else rec["loc"].size
                rows += per * n_out
            steps_done += 1
            if spent + time.perf_counter() - t0 > budget_s:
                break
        spent += time.perf_counter() - t0
        passes += 1
    # the oracle runs one thread per request shard: at most n of them
    which = (f"all {cfg.n_req} requests" if n == cfg.n_req
             else f"requests 0..{n - 1} of {cfg.n_req}")
    return {"value": round(rows / spent, 1), "unit": "rows/s",
            "cores": int(min(src.threads, n)),
            "kind": "oracle",
            "sample": f"{cfg.name}: {passes} pass(es) over decode steps 0..{total_steps - 1} of "
                      f"{which} from a fresh state, {steps_done} steps, "
                      f"{spent:.1f} s of oracle time"}


def host_link_gbs(torch, nbytes=1 << 30, reps=5):
    """Pinned host -> device copy rate (hipMemcpyAsync through torch)."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src, non_blocking=True)
        b.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, dst
    return best


# Counter-based memory traffic of the gathering kernels (the resident gather
# alone, the step kernel), one summary per workload and kernel.  A summary
# records the hash of the kernel sources it was taken with; once they change
# the figure no longer applies and is dropped.
TRAFFIC_PROFILES = os.path.join(ROOT, "profiles", "*_traffic.md")
GATHER_SOURCES = [os.path.join(ROOT, "hierarchical_sparse_kv_resolve_amd", "csrc", name)
                  for name in ("gather.hip", "gather_body.h", "rows.h", "step.hip",
                               "resolve_body.h", "block.h")]


def gather_source_hash():
    """sha256 over the gathering kernels' source files, in order."""
    import hashlib
    h = hashlib.sha256()
    for path in GATHER_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_records():
    """The recorded counter summaries: one dict of fields per profile file."""
    import glob
    out = []
    for path in sorted(glob.glob(TRAFFIC_PROFILES)):
        with open(path) as f:
            out.append(dict(re.findall(r"^(\w+): (\S+)$", f.read(), re.M)))
    return out


def recorded_traffic(workload, schedule, kernel="gather_kernel"):
    """Bytes per launch of `kernel` (gather_kernel or fused_gather_kernel)
    measured by counters for this workload and schedule on the current
    source of those kernels, or None."""
    source = gather_source_hash()
    for fields in traffic_records():
        if (fields.get("workload") == workload and fields.get("schedule") == schedule
                and fields.get("kernel", "gather_kernel") == kernel
                and fields.get("source_sha256") == source):
            try:
                return int(fields["traffic_bytes_per_launch"])
            except (KeyError, ValueError):
                return None
    return None


def copy_calibration(torch, nbytes=1 << 30, reps=3):
    """Plain device-to-device copies of nbytes, for scaling FETCH_SIZE/WRITE_SIZE:
    torch's copy_ (the runtime's blit kernel) and an elementwise bitwise_not
    (one read and one write of every byte)."""
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    for _ in range(reps):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps,
                      "kernels": ["copy_", "bitwise_not"]}), flush=True)


def device_copy_gbs(torch, nbytes=4 << 30, reps=3):
    """Best rate (read + write bytes) of a plain device-to-device copy of
    nbytes through torch (the runtime's copy kernel), far larger than the
    last-level cache: what a streaming copy reaches on this HBM."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = max(best, 2 * nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, dst
    return best


def zero_copy_read_gbs(torch, gpu, reps=3):
    """Sequential zero-copy read rate of the pinned host stores by the refill
    kernel itself: every request's first B host rows, in order, into its B hot
    slots, all payload layers in one call; best of `reps`.  It overwrites the
    hot caches, so it runs after the timed pass has been checked."""
    from hierarchical_sparse_kv_resolve_amd import kvr
    cfg, n = gpu.cfg, gpu.n
    B = min(cfg.B, gpu.inputs.host_rows)
    fills = torch.zeros((n, cfg.B, 2), dtype=torch.int32, device="cuda")
    j = torch.arange(B, dtype=torch.int32, device="cuda")
    fills[:, :B, 0] = j
    fills[:, :B, 1] = j
    fc = torch.full((n,), B, dtype=torch.int32, device="cuda")
    layers = list(range(gpu.nl))
    nbytes = n * B * cfg.R * len(layers)
    best = 0.0
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        gpu.ctx.reuse_locations(kvr.REUSE_DISTINCT_PAYLOAD, layers, n, None, gpu.loc[0], None,
                                None, cfg.sel_cap, fills, fc)
        b.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    return best


def load_step_scenario(torch, args):
    """The load-step on/off experiment on the GLM-style shape: a pool with
    spare pages; after a low-load phase an admission needs the spare pages
    plus four requests' worth of optional pages (reclaimed whole, in request
    order, with host backup); it drains after the pressure phase and bounded
    round-robin refill then repopulates the pool (refill continues into the
    last phase while free pages and not-ready pages remain).  Reports, per phase, the
    share of selected rows fetched from host memory and the throughput, and
    the same steps with no optional residency at all (every page on the host)
    as the baseline.  The residency plan does not depend on device results, so
    it is made up front by the library's host policy and its page lists are
    staged on the device before timing; each step then issues its page moves
    and its decode step on one stream."""
    from hierarchical_sparse_kv_resolve_amd import kvr
    from hierarchical_sparse_kv_resolve_amd.runner import GpuRun
    from synth import FULL, Inputs, payload_np
    W, L1, L2, L3, L4 = args.warmup, 12, 16, 112, 16
    total = W + L1 + L2 + L3 + L4
    base = FULL[2].with_(steps=total, pool_spare=256)
    t2, t3 = W + L1 + L2, W + L1 + L2 + L3
    phases = [("low_load", W, W + L1), ("pressure", W + L1, t2), ("refill", t2, t3),
              ("after_refill", t3, total)]

    def run_case(cfg, residency):
        inputs = Inputs(cfg, max_new=total)
        gpu = GpuRun(inputs)
        gpu.stage(range(total))
        plan = {}
        if residency:
            pol = kvr.Residency(inputs.page_map, cfg.full_pages, cfg.pool_pages)
            need = cfg.pool_spare + 4 * cfg.ready_pages - cfg.ready_pages // 2
            ok, reclaim, handle = pol.admit(need, list(range(cfg.n_req)))
            assert ok
            plan[W + L1] = ("reclaim", reclaim)
            for s in range(W + L1 + L2, total):
                if s == W + L1 + L2:
                    pol.release(handle)
                plan[s] = ("restore", pol.refill(args.refill_bound))
            pol.close()
        dev = []  # page lists staged on the device
        for s in sorted(plan):
            kind, lst = plan[s]
            cols = list(zip(*lst)) if lst else []
            arrs = [torch.tensor(list(c), dtype=torch.int32, device="cuda") for c in cols]
            n = len(lst)
            aux = torch.full((max(1, n),), -1, dtype=torch.int32, device="cuda")
            st = torch.zeros(max(1, n), dtype=torch.int32, device="cuda")
            plan[s] = (kind, n, arrs, aux, st)
            dev.append(st)
        for s in range(W):
            gpu.step(s, prefetch_groups=2)
        torch.cuda.synchronize()
        out = {}
        moved_bytes = 0
        for name, lo, hi in phases:
            before = gpu.stats_dict()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            pages = 0
            for s in range(lo, hi):
                if s in plan:
                    kind, n, arrs, aux, st = plan[s]
                    if n and kind == "reclaim":
                        gpu.ctx.reclaim_pages(n, arrs[0], arrs[1], aux, st)
                    elif n:
                        gpu.ctx.restore_pages(n, arrs[0], arrs[1], arrs[2], st)
                    pages += n
                gpu.step(s, prefetch_groups=2)
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            after = gpu.stats_dict()
            d = {k: after[k] - before[k] for k in after}
            found = max(1, d["tail"] + d["page"] + d["hit"] + d["miss"])
            steps = hi - lo
            rows = steps * cfg.n_req * cfg.k * cfg.payload_layers
            out[name] = {"steps": steps, "ms_per_step": round(ms / steps, 4),
                         "rows_per_s": round(rows / (ms * 1e-3), 1),
                         "host_share": round(d["miss"] / found, 4),
                         "tail_or_page_share": round((d["tail"] + d["page"]) / found, 4),
                         "hot_share": round(d["hit"] / found, 4),
                         "pages_moved": pages,
                         "page_bytes_per_step": int(pages * cfg.P * cfg.R * cfg.payload_layers
                                                    / steps)}
        for st in dev:
            if (st.cpu().numpy() != 0).any():
                raise SystemExit("a page move reported an error")
        for g in range(cfg.groups):
            if (gpu.status[g].cpu().numpy() != 0).any():
                raise SystemExit("resolve failed")
        last = total - 1
        sel = inputs.selections(last, 0)[:, 0, :]
        rec = gpu.group(0)
        for r in range(cfg.n_req):
            j = np.arange(0, 64)
            for l, o in enumerate(rec["out"]):
                if not np.array_equal(o[r, j], payload_np(l, r, sel[r, j], cfg.R, cfg.seed)):
                    raise SystemExit("gathered bytes differ from the payload closed form")
        gpu.close()
        return out

    log("load step: optional residency on")
    on = run_case(base, True)
    log("load step: no optional residency (every page on the host)")
    off = run_case(base.with_(ready_frac=0.0, pool_spare=0), False)
    line = {"metric": "load-step scenario: host-fetched share of selected rows and rows/s per phase",
            "scenario": "load_step", "n_gpus": 1, "data": "synthetic", "dtype": "u8",
            "config": {"workload": base.name, "pool_spare_pages": base.pool_spare,
                       "ready_pages_per_request": base.ready_pages,
                       "admission_pages": base.pool_spare + 4 * base.ready_pages
                       - base.ready_pages // 2,
                       "refill_bound_pages_per_step": args.refill_bound,
                       "phases": {name: [lo, hi] for name, lo, hi in phases}},
            "residency_on": on, "residency_off": off}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the resolver keeps each request's state on "
              "one device and the library has no multi-GPU path (--gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.scenario == "load_step":
        load_step_scenario(torch, args)
        return
    from hierarchical_sparse_kv_resolve_amd.runner import GpuRun
    from synth import FULL, Inputs

    c = int(args.workload[1])
    K, W = args.steps, args.warmup
    total = K + W
    cfg = FULL[c].with_(steps=total)
    if args.hot_slots:
        cfg = cfg.with_(B=args.hot_slots)
    inputs = Inputs(cfg, max_new=total)
    log(f"workload {cfg.name}: staging {total} steps")
    gpu = GpuRun(inputs, step_buffers=args.step_buffers)
    gpu.stage(range(total))
    log("staged; warming up")
    counts = rows_per_group(inputs, range(W, total))
    pg = args.prefetch_groups
    pg = int(pg) if "," not in pg else tuple(int(x) for x in pg.split(","))
    schedule = auto_schedule(cfg) if args.schedule == "auto" else args.schedule
    kw = dict(prefetch_groups=pg, **schedule_kwargs(schedule))
    fused, merged = kw["fused"], kw["merged"]
    no_graph = args.no_graph
    if fused and cfg.reuse != "distinct" and not no_graph:
        # its graph capture is disabled (GpuRun.capture): timed eagerly
        log("the fused schedule of one physical source runs eagerly (no graph)")
        no_graph = True
    for s in range(W):
        gpu.step(s, **kw)
    gpu.finish()
    torch.cuda.synchronize()
    snap = gpu.snapshot()
    stats_before = gpu.stats_dict()

    # Pass 1 (eager, same steps, same launches): the library records the start
    # and end of every kernel dispatch (events on the dispatches themselves;
    # events cannot be recorded inside a graph); the launches are serialized
    # so each recorded duration is one kernel running alone.
    gpu.ctx.timing_begin(64 * K + 64)
    for s in range(W, total):
        gpu.step(s, prefetch_groups=pg, serialize=True, fused=fused)
    launches = launch_means_ms(gpu.ctx.timing_end())
    torch.cuda.synchronize()
    if fused:
        # Pass 1b: the timed pass runs the fill and the resident gather as one
        # launch; time that launch too, with the launches of the timed pass
        # (one stream for distinct payloads; for one physical source each
        # fused launch overlaps the next layer's resolve, as when timed).
        gpu.restore(snap)
        gpu.ctx.timing_begin(64 * K + 64)
        for s in range(W, total):
            gpu.step(s, **kw)
        gpu.finish()
        rec = launch_means_ms(gpu.ctx.timing_end())
        torch.cuda.synchronize()
        launches["fused"] = rec.get("fused", [])
        if merged:
            # each launch but the last gathers one selection beside the next resolve
            launches["step"] = rec.get("step", [])
        # Pass 1c: the plain calls over the same steps (resolve_rows with its
        # host fill, then one gather_rows of every row), so that the gather
        # call of the boundary is timed on its own as well
        gpu.restore(snap)
        gpu.ctx.timing_begin(64 * K + 64)
        for s in range(W, total):
            gpu.step(s, serialize=True)
        gpu.finish()
        plain_gathers = launch_means_ms(gpu.ctx.timing_end()).get("gather", [])
        torch.cuda.synchronize()
    if not no_graph:
        gpu.restore(snap)
        graph = gpu.capture(range(W, total), **kw)
        torch.cuda.synchronize()
        log("captured the timed steps into one graph")

    # Pass 2 (timed): the K decode steps from the same starting state, run
    # `repeats` times (state restored before each); every run is checked and
    # the median is reported.
    from synth import payload_np

    def check_run():
        # every request of every timed call must have resolved
        for g in range(cfg.groups):
            st = gpu.status[g].cpu().numpy()
            if (st != 0).any():
                raise SystemExit(f"resolve failed: status {st.tolist()}")
        if ((gpu.gather_status.cpu().numpy() != 0).any()
                or (gpu.append_status.cpu().numpy() != 0).any()):
            raise SystemExit("gather or append reported an error")
        # spot check of the last step against the payload closed form
        last = total - 1
        rec = gpu.group(cfg.groups - 1)
        sel = inputs.selections(last, cfg.groups - 1)
        rows_src = rec["union"] if cfg.q > 1 else sel[:, 0, :]
        for r in range(0, cfg.n_req, max(1, cfg.n_req // 4)):
            j = np.arange(0, 64)
            for l, out in enumerate(rec["out"]):
                if not np.array_equal(out[r, j], payload_np(l, r, rows_src[r, j], cfg.R, cfg.seed)):
                    raise SystemExit("gathered bytes differ from the payload closed form")

    walls, gpu_mss = [], []
    for rep in range(max(1, args.repeats)):
        if rep > 0 or no_graph:
            gpu.restore(snap)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        if no_graph:
            for s in range(W, total):
                gpu.step(s, **kw)
            gpu.finish()
        else:
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
        gpu_mss.append(start.elapsed_time(end))
        log(f"run {rep}: timed {K} steps in {walls[-1] * 1e3:.3f} ms")
        check_run()
    wall_s = float(np.median(walls))
    gpu_ms = float(np.median(gpu_mss))

    n_out = cfg.payload_layers if cfg.reuse == "distinct" else 1
    rows_total = sum(counts.values()) * n_out
    value = rows_total / wall_s
    # the same per (query, selected row) entry: q*k per request for a verify
    # block, whose rows are gathered once per union row
    sel_entries = K * cfg.groups * cfg.n_req * cfg.q * cfg.k * n_out

    stats_all = gpu.stats_dict()
    stats = {kk: stats_all[kk] - stats_before[kk] for kk in stats_all}
    # Algorithmic bytes per launch (rows already resident in HBM and pinned
    # host memory when timing starts):
    #   gather (all rows, or the resident rows of the fused schedule): each
    #     moved row R read + R written per payload layer, plus one 4-byte
    #     location word per entry;
    #   fused launch: every entry's row written to the output (2R per layer
    #     in HBM: a resident row is read and written; a fresh row crosses the
    #     host link once, R, and is written to its hot slot and the output),
    #     plus the location word of every entry and the selection entry of
    #     every fresh one;
    #   refill: each filled row R over the host link and R written, per layer.
    entries = sum(counts.values())
    fresh = stats["miss"]
    g_list = launches.get("gather", [])
    gather_calls = len(g_list)
    moved = entries - fresh if fused else entries
    bytes_gather = (moved * 2 * cfg.R * n_out + entries * 4) / max(1, gather_calls)
    g_ms = sum(g_list) / max(1, gather_calls)
    g_gbs = bytes_gather / (g_ms * 1e-3) / 1e9 if g_ms > 0 else 0.0
    dev_copy = device_copy_gbs(torch)
    gather_alone = {"kernel": "gather_kernel<resident>" if fused else "gather_kernel<all>",
                    "achieved": round(g_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(g_gbs / HBM_PEAK_GBS, 4),
                    "traffic": recorded_traffic(cfg.name, "fused" if fused
                                                else f"prefetch:{args.prefetch_groups}"),
                    "bytes_per_launch": int(bytes_gather), "launch_us": round(g_ms * 1e3, 2),
                    "device_copy_gbs": round(dev_copy, 1),
                    "frac_of_device_copy": round(g_gbs / dev_copy, 4),
                    "timing": "start/end events of each gather dispatch (hipExtLaunchKernel) in "
                              "an eager pass over the same timed steps from the same starting "
                              "state, no two kernels overlapping"
                              + ("; in the timed pass this gather is the resident part of the "
                                 "fused launch" if fused else "")}

    # host refill path: every fill is fetched once per payload layer (all layers
    # replay the fills for shared indices with distinct payloads)
    fill_layers = cfg.payload_layers if cfg.reuse == "distinct" else 1
    host_bytes = stats["fill"] * cfg.R * fill_layers
    fill_calls = launches.get("refill", [])
    fill_s = sum(fill_calls) * 1e-3
    copy_gbs = host_link_gbs(torch)
    seq_gbs = zero_copy_read_gbs(torch, gpu)
    link = max(copy_gbs, seq_gbs)
    refill_gbs = host_bytes / fill_s / 1e9 if fill_s > 0 else None
    host_link = {"refill_gbs": round(refill_gbs, 1) if refill_gbs else None,
                 "pinned_h2d_copy_gbs": round(copy_gbs, 1),
                 "zero_copy_seq_read_gbs": round(seq_gbs, 1),
                 "frac": round(refill_gbs / link, 4) if refill_gbs else None,
                 "host_bytes_per_step": int(host_bytes / K),
                 "refill_calls_per_step": len(fill_calls) / K}

    # The roofline is that of the kernel that takes most of the timed pass.
    if fused:
        # the launches that gather: fused ones, and with the merged schedule
        # the step launches (a gather beside the next resolve)
        f_list = launches.get("step", []) + launches.get("fused", [])
        n_launch = max(1, len(f_list))
        d_ms = sum(f_list) / n_launch
        d_host = n_out * fresh * cfg.R / n_launch
        d_hbm = (n_out * entries * 2 * cfg.R + entries * 4 + fresh * 4) / n_launch
        d_kernel = "step_kernel" if merged else "fused_gather_kernel"
        d_timing = ("start/end events of each gathering dispatch in an eager pass of the timed "
                    "pass's own launches (same streams and overlaps) over the same steps from "
                    "the same starting state")
    elif fill_calls and sum(fill_calls) >= sum(g_list):
        n_launch = len(fill_calls)
        d_ms = fill_s * 1e3 / n_launch
        d_host = host_bytes / n_launch
        d_hbm = (host_bytes + stats["fill"] * 8 * fill_layers) / n_launch
        d_kernel = "refill_kernel"
        d_timing = ("start/end events of each refill dispatch in an eager pass over the same "
                    "timed steps from the same starting state, no two kernels overlapping")
    else:
        n_launch, d_ms, d_host, d_hbm = gather_calls, g_ms, 0.0, bytes_gather
        d_kernel, d_timing = gather_alone["kernel"], gather_alone["timing"]
    d_s = max(d_ms, 1e-9) * 1e-3
    hbm_gbs = d_hbm / d_s / 1e9
    host_gbs = d_host / d_s / 1e9
    hbm_part = {"achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": int(d_hbm)}
    if d_host > 0:
        roofline = {"bound": "host_link", "achieved": round(host_gbs, 1),
                    "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                    "frac": round(host_gbs / HOST_LINK_PEAK_GBS, 4),
                    "traffic": recorded_traffic(cfg.name, schedule if fused else
                                                f"prefetch:{args.prefetch_groups}", d_kernel),
                    "kernel": d_kernel, "bytes_per_launch": int(d_host),
                    "launch_us": round(d_ms * 1e3, 2), "launches": n_launch,
                    "measured_link_gbs": round(link, 1),
                    "frac_of_measured_link": round(host_gbs / link, 4),
                    "hbm": hbm_part, "timing": d_timing}
    else:
        roofline = dict(hbm_part, bound="hbm", kernel=d_kernel, launch_us=round(d_ms * 1e3, 2),
                        launches=n_launch, traffic=gather_alone["traffic"], timing=d_timing)
    roofline["gather_alone"] = gather_alone
    if fused and plain_gathers:
        # every row of every entry moved (fresh rows from their hot slots)
        a_bytes = (entries * 2 * cfg.R * n_out + entries * 4) / len(plain_gathers)
        a_ms = sum(plain_gathers) / len(plain_gathers)
        a_gbs = a_bytes / (a_ms * 1e-3) / 1e9
        roofline["gather_rows"] = {
            "kernel": "gather_kernel<all>", "achieved": round(a_gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(a_gbs / HBM_PEAK_GBS, 4),
            "bytes_per_launch": int(a_bytes), "launch_us": round(a_ms * 1e3, 2),
            "launches": len(plain_gathers),
            "frac_of_device_copy": round(a_gbs / dev_copy, 4),
            "timing": "start/end events of each gather_rows dispatch in an eager pass of the "
                      "plain calls (resolve_rows with its host fill, then gather_rows of every "
                      "row) over the same timed steps from the same starting state, no two "
                      "kernels overlapping"}

    found = max(1, stats["tail"] + stats["page"] + stats["hit"] + stats["miss"])
    split = {"step1_tail_or_page": round((stats["tail"] + stats["page"]) / found, 4),
             "step2_hot_hit": round(stats["hit"] / found, 4),
             "step3_host": round(stats["miss"] / found, 4)}
    per_call_us = {name: round(sum(v) / len(v) * 1e3, 2) for name, v in launches.items()}
    line = {
        "metric": "selected rows resolved+gathered/sec and achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(value, 1), "unit": "rows/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(wall_s * 1e3 / K, 4), "higher_is_better": True, "scaling": "weak",
        "repeats": len(walls), "ms_per_step_runs": [round(w * 1e3 / K, 4) for w in walls],
        "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": cfg.name, "schedule": schedule,
                   "prefetch_groups": None if fused else args.prefetch_groups,
                   "launch": "eager" if no_graph else "hip_graph", "n_req": cfg.n_req, "history_rows": cfg.H,
                   "row_bytes": cfg.R, "page_rows": cfg.P, "tail_rows": cfg.T,
                   "ready_frac": cfg.ready_frac, "hot_slots": cfg.B, "top_k": cfg.k,
                   "verify_queries": cfg.q, "payload_layers": cfg.payload_layers,
                   "model_layers": cfg.model_layers, "resolving_layers": cfg.groups,
                   "selection": cfg.sel, "zipf_s": cfg.zipf_s, "parallelism": "none"},
        "roofline": roofline,
        "gpu_ms_per_step": round(gpu_ms / K, 4),
        "selection_entries_per_s": round(sel_entries / wall_s, 1),
        "per_call_us": per_call_us,
        "resolution_split": split,
        "host_link": host_link,
    }
    gpu.close()
    if not args.no_cpu_baseline:
        log("timing the oracle on the host cores")
        line["cpu_baseline"] = cpu_baseline(cfg, total, args.cpu_budget_s,
                                            n_reqs=args.cpu_requests)
        line["cpu_baseline"]["cpu_model"] = cpu_model()
        one = cpu_baseline(cfg, total, args.cpu_budget_s / 2, min_s=4.0, threads=1,
                           n_reqs=args.cpu_requests)
        line["cpu_baseline"]["single_core"] = {"value": one["value"], "unit": one["unit"],
                                               "sample": one["sample"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
