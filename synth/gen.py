"""Seeded synthetic inputs shared by the GPU path and the CPU reference.

Everything here is input generation: page readiness, physical page ids, row
payload bytes, new decoded rows and per-step selections.  None of the
resolver's arithmetic lives here.

Readings of the shapes (the pages leave these open):
  * ready pages: round(ready_frac * complete pages) per request, chosen without
    replacement; physical ids are one seeded permutation of the global pool;
  * resident-first admission defers host backup, so a ready page has no host
    copy (its host rows hold the 0xDB poison); every other imported row and
    every decoded row has one;
  * the tail initially holds the last T imported rows;
  * "mix" selection: floor(frac * k) distinct rows from the most recent window
    plus the rest distinct over the whole history, shuffled;
  * "zipf" selection: k distinct rows drawn by weighted sampling without
    replacement, weight (rank + 1) ** -s with rank = L - 1 - pos (recency rank),
    by the exponential-race method of Efraimidis & Spirakis (2006), shuffled;
  * "uniform": k distinct rows uniform over [0, L), shuffled;
  * verify block: query 0 as above; each other query keeps a random
    floor(shared_frac * k) subset of query 0 and adds k minus that many fresh
    rows outside query 0 drawn from the same distribution.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import Workload

POISON_HOST = 0xDB      # host rows without a host copy
POISON_HOT = 0xCD       # hot slots never filled
POISON_OUT = 0xEE       # gather outputs before the gather
POISON_FREE_PAGE = 0xFA  # optional-pool pages no request holds

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build_lib() -> str:
    """Compile the payload filler (plain C, host only)."""
    src = os.path.join(_HERE, "payload.c")
    cmd = ["gcc", "-O3", "-march=x86-64-v2", "-fPIC", "-shared", "-pthread", src, "-o", _LIB_PATH]
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_fill_segments.restype = ctypes.c_int
        lib.synth_fill_segments.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.c_uint64, ctypes.c_int32]
        _lib = lib
    return _lib


SEG_DTYPE = np.dtype([("dst", np.uint64), ("n_rows", np.int64), ("stride", np.int64),
                      ("layer", np.int64), ("req", np.int64), ("pos0", np.int64)])


def n_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------------------
# payload closed form, numpy edition (used by tests to check gathered bytes)

_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_G = np.uint64(0x9E3779B97F4A7C15)


def mix64_np(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = x.astype(np.uint64) + _G
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def payload_np(layer, req, pos, row_bytes: int, seed: int) -> np.ndarray:
    """Bytes of rows (layer, req, pos) -> uint8 [..., row_bytes].  Broadcasts."""
    layer = np.asarray(layer, dtype=np.uint64)
    req = np.asarray(req, dtype=np.uint64)
    pos = np.asarray(pos, dtype=np.uint64)
    w = np.arange(row_bytes // 8, dtype=np.uint64)
    key = ((layer << np.uint64(56)) | (req << np.uint64(40)) | (pos << np.uint64(16)))[..., None] | w
    words = mix64_np(np.uint64(seed) ^ key)
    return words.astype("<u8").view(np.uint8).reshape(*words.shape[:-1], row_bytes)


def fill_segments(segs: np.ndarray, row_bytes: int, seed: int) -> None:
    segs = np.ascontiguousarray(segs, dtype=SEG_DTYPE)
    rc = _load().synth_fill_segments(segs.ctypes.data, len(segs), row_bytes, seed, n_threads())
    if rc != 0:
        raise ValueError("synth_fill_segments rejected its arguments")


def _seg(dst: np.ndarray, n_rows: int, stride: int, layer: int, req: int, pos0: int):
    return (dst.ctypes.data, n_rows, stride, layer, req, pos0)


# ---------------------------------------------------------------------------


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


class Inputs:
    """All seeded inputs of one workload.

    The caller owns the memory that payload is written into, so the GPU side can
    fill pinned host memory and the CPU reference its own private arrays.
    `max_new` is the number of decoded rows each request may append.
    """

    def __init__(self, cfg: Workload, max_new: int | None = None):
        self.cfg = cfg
        self.max_new = cfg.steps if max_new is None else int(max_new)
        self.host_rows = cfg.H + self.max_new
        self.payload_seed = cfg.seed
        c = cfg
        page_map = np.full((c.n_req, c.n_pages), -1, dtype=np.int32)
        host_valid = np.ones((c.n_req, c.n_pages), dtype=np.uint8)
        perm = _rng(c.seed, 2).permutation(c.pool_pages).astype(np.int64)
        owner_req = np.full(c.pool_pages, -1, dtype=np.int64)    # -1: a free page
        owner_page = np.full(c.pool_pages, -1, dtype=np.int64)
        nxt = 0
        for r in range(c.n_req):
            ready = np.sort(_rng(c.seed, 1, r).choice(c.full_pages, size=c.ready_pages, replace=False))
            phys = perm[nxt:nxt + c.ready_pages]
            nxt += c.ready_pages
            page_map[r, ready] = phys.astype(np.int32)
            host_valid[r, ready] = 0
            owner_req[phys] = r
            owner_page[phys] = ready
        self.page_map = page_map
        self.host_valid = host_valid
        self.owner_req = owner_req
        self.owner_page = owner_page

    # -- payload ---------------------------------------------------------
    def _reqs(self, reqs):
        return list(range(self.cfg.n_req)) if reqs is None else [int(r) for r in reqs]

    def fill_host(self, layer: int, dst: np.ndarray, reqs=None) -> None:
        """dst: uint8 [n][H + max_new][R] for requests `reqs` (default: all), in
        any memory.  Imported rows with a host copy get their payload; all other
        rows the host poison."""
        c = self.cfg
        reqs = self._reqs(reqs)
        assert dst.shape == (len(reqs), self.host_rows, c.R) and dst.dtype == np.uint8
        assert dst.flags.c_contiguous
        dst.fill(POISON_HOST)
        segs = []
        for i, r in enumerate(reqs):
            valid = self.host_valid[r]
            p = 0
            while p < c.n_pages:
                if not valid[p]:
                    p += 1
                    continue
                q = p
                while q < c.n_pages and valid[q]:
                    q += 1
                lo, hi = p * c.P, min(q * c.P, c.H)
                segs.append(_seg(dst[i, lo], hi - lo, c.R, layer, r, lo))
                p = q
        fill_segments(np.array(segs, dtype=SEG_DTYPE), c.R, self.payload_seed)

    def fill_pool(self, layer: int, dst: np.ndarray) -> None:
        """dst: uint8 [pool_pages][P][R]; free pages get the free-page poison."""
        c = self.cfg
        assert dst.shape == (c.pool_pages, c.P, c.R) and dst.dtype == np.uint8
        assert dst.flags.c_contiguous
        if c.pool_pages == 0:
            return
        free = self.owner_req < 0
        if free.any():
            dst[free] = POISON_FREE_PAGE
        segs = [_seg(dst[ph], c.P, c.R, layer, int(self.owner_req[ph]), int(self.owner_page[ph]) * c.P)
                for ph in range(c.pool_pages) if self.owner_req[ph] >= 0]
        if not segs:
            return
        fill_segments(np.array(segs, dtype=SEG_DTYPE), c.R, self.payload_seed)

    def fill_tail(self, layer: int, dst: np.ndarray, reqs=None) -> None:
        """dst: uint8 [n][T][R]: the last T imported rows, at pos mod T."""
        c = self.cfg
        reqs = self._reqs(reqs)
        assert dst.shape == (len(reqs), c.T, c.R) and dst.dtype == np.uint8
        dst.fill(POISON_HOST)
        if c.T == 0:
            return
        segs = []
        for i, r in enumerate(reqs):
            pos = max(0, c.H - c.T)
            while pos < c.H:
                run = min(c.H - pos, c.T - pos % c.T)
                segs.append(_seg(dst[i, pos % c.T], run, c.R, layer, r, pos))
                pos += run
        fill_segments(np.array(segs, dtype=SEG_DTYPE), c.R, self.payload_seed)

    def new_rows(self, step: int, reqs=None) -> np.ndarray:
        """Row appended at decode step `step`: uint8 [payload_layers][n][R],
        the payload of position H + step."""
        c = self.cfg
        lay = np.arange(c.payload_layers)[:, None]
        req = np.asarray(self._reqs(reqs))[None, :]
        return np.ascontiguousarray(payload_np(lay, req, c.H + step, c.R, self.payload_seed))

    # -- selections ------------------------------------------------------
    def length_at(self, step: int) -> int:
        """Rows per request after the step's append (one row per step)."""
        return self.cfg.H + step + 1

    def _zipf(self, rng, L: int, k: int, exclude=None) -> np.ndarray:
        rank = (L - 1) - np.arange(L, dtype=np.float64)
        keys = rng.standard_exponential(L) * np.power(rank + 1.0, self.cfg.zipf_s)
        if exclude is not None and len(exclude):
            keys[exclude] = np.inf
        k = min(k, L if exclude is None else L - len(exclude))
        pick = np.argpartition(keys, k - 1)[:k] if k > 0 else np.empty(0, dtype=np.int64)
        return np.sort(pick)

    def _one_query(self, rng, L: int) -> np.ndarray:
        c = self.cfg
        k = min(c.k, L)
        if c.sel == "uniform":
            rows = np.sort(rng.choice(L, size=k, replace=False))
        elif c.sel == "zipf":
            rows = self._zipf(rng, L, k)
        elif c.sel == "mix":
            lo = max(0, L - c.mix_recent)
            n_recent = min(int(np.floor(c.mix_recent_frac * k)), L - lo)
            recent = lo + rng.choice(L - lo, size=n_recent, replace=False)
            rest_pool = np.setdiff1d(np.arange(L), recent, assume_unique=True)
            rest = rng.choice(rest_pool, size=k - n_recent, replace=False)
            rows = np.sort(np.concatenate([recent, rest]))
        else:
            raise ValueError(c.sel)
        return rows

    def selections(self, step: int, group: int = 0, reqs=None) -> np.ndarray:
        """Selections of one resolving layer at one step: int32 [n][q][k]."""
        c = self.cfg
        L = self.length_at(step)
        reqs = self._reqs(reqs)
        out = np.empty((len(reqs), c.q, min(c.k, L)), dtype=np.int32)
        for i, r in enumerate(reqs):
            rng = _rng(c.seed, 3, step, group, r)
            q0 = self._one_query(rng, L)
            out[i, 0] = rng.permutation(q0)
            n_shared = int(np.floor(c.shared_frac * len(q0)))
            for qi in range(1, c.q):
                keep = rng.choice(q0, size=n_shared, replace=False)
                fresh = self._zipf(rng, L, len(q0) - n_shared, exclude=q0)
                out[i, qi] = rng.permutation(np.concatenate([keep, fresh]))
        return out
