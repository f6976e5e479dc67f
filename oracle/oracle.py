"""Python handle on the CPU reference (oracle) of the sparse KV row resolver.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline use it; the product path never imports it.  It shares no code with
the GPU library.  The rules themselves live in kvr_oracle.c (plain C); this
file only holds the state arrays and marshals calls.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liborc.so")

OK = 0
E_ARG = -1
E_RANGE = -2
E_CAPACITY = -3
E_NO_HOST_COPY = -4
E_STATE = -6

INVALID = 0xFFFFFFFF
FRESH = 1 << 29  # hot-cache location word: copied from host in this call
STAT_NAMES = ("calls", "tail", "page", "hit", "miss", "fill", "host_bytes", "error")

_P = ctypes.c_void_p
_I = ctypes.c_int32


class _Source(ctypes.Structure):
    _fields_ = [("n_req", _I), ("n_layers", _I), ("H", _I), ("max_new", _I), ("P", _I),
                ("T", _I), ("B", _I), ("R", _I), ("pool_pages", ctypes.c_int64),
                ("L", _P), ("page_map", _P), ("host_valid", _P), ("tag", _P), ("stamp", _P),
                ("clock", _P), ("tail", _P), ("pool", _P), ("hot", _P), ("host", _P)]


def build_lib() -> str:
    src = os.path.join(_HERE, "kvr_oracle.c")
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-pthread", "-Wall",
                    src, "-o", LIB_PATH], check=True)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build_lib()
        L = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int32
        sigs = {
            "orc_resolve": [P, I, P, P, P, I, I, P, P, P, P, P, I],
            "orc_gather": [P, I, I, P, P, P, I, P, P, I],
            "orc_replay": [P, I, I, P, P, P, P, I],
            "orc_dedup": [P, I, I, I, P, P, P, P, I],
            "orc_append": [P, I, P, P, P, I],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.restype = None
            fn.argtypes = args
        for name, args in {"orc_reclaim_pages": [P, I, P, P, P, P],
                           "orc_restore_pages": [P, I, P, P, P, P]}.items():
            fn = getattr(L, name)
            fn.restype = None
            fn.argtypes = args
        L.orc_check_one.restype = ctypes.c_int
        L.orc_check_one.argtypes = [P, I]
        _lib = L
    return _lib


def _p(a) -> int:
    return 0 if a is None else a.ctypes.data


def default_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 1


class OracleSource:
    """One KV source (its metadata and payload layers) as plain numpy arrays.

    host[l] must be a private uint8 [n_req][H + max_new][R] array; pool[l] is
    written only by restore_pages.  All mutable state is owned here.
    """

    def __init__(self, *, n_req, n_layers, H, max_new, P, T, B, R, page_map, host_valid,
                 tail, pool, host, threads=None):
        self.n_req, self.n_layers, self.H, self.max_new = n_req, n_layers, H, max_new
        self.P, self.T, self.B, self.R = P, T, B, R
        self.threads = threads or default_threads()
        n_pages = -(-H // P)
        self.page_map = np.ascontiguousarray(page_map, dtype=np.int32).reshape(n_req, n_pages)
        self.host_valid = np.ascontiguousarray(host_valid, dtype=np.uint8).reshape(n_req, n_pages)
        self.L = np.full(n_req, H, dtype=np.int32)
        self.tag = np.full((n_req, B), -1, dtype=np.int32)
        self.stamp = np.zeros((n_req, B), dtype=np.uint32)
        self.clock = np.zeros(n_req, dtype=np.uint32)
        self.tail = [np.ascontiguousarray(t) for t in tail]
        self.pool = [np.ascontiguousarray(p) for p in pool]
        self.host = list(host)
        self.hot = [np.full((n_req, B, R), 0xCD, dtype=np.uint8) for _ in range(n_layers)]
        pool_pages = self.pool[0].shape[0] if self.pool else 0
        for l in range(n_layers):
            assert self.tail[l].shape == (n_req, T, R)
            assert self.pool[l].shape == (pool_pages, P, R)
            assert self.host[l].shape == (n_req, H + max_new, R) and self.host[l].flags.c_contiguous
        self.stats = np.zeros(len(STAT_NAMES), dtype=np.uint64)
        self._ptrs = {}
        for name in ("tail", "pool", "hot", "host"):
            arr = (ctypes.c_void_p * max(1, n_layers))(*[a.ctypes.data for a in getattr(self, name)])
            self._ptrs[name] = arr
        self._src = _Source(n_req, n_layers, H, max_new, P, T, B, R, pool_pages,
                            _p(self.L), _p(self.page_map), _p(self.host_valid), _p(self.tag),
                            _p(self.stamp), _p(self.clock),
                            ctypes.cast(self._ptrs["tail"], _P), ctypes.cast(self._ptrs["pool"], _P),
                            ctypes.cast(self._ptrs["hot"], _P), ctypes.cast(self._ptrs["host"], _P))

    @property
    def src(self):
        return ctypes.byref(self._src)

    def _req(self, req_ids, n):
        if req_ids is None:
            return None
        r = np.ascontiguousarray(req_ids, dtype=np.int32)
        assert r.shape == (n,)
        return r

    # -- calls ---------------------------------------------------------------
    def append(self, new_rows: np.ndarray, req_ids=None) -> np.ndarray:
        """new_rows: uint8 [n_layers][n_req][R]. Returns per-request status."""
        rows = np.ascontiguousarray(new_rows, dtype=np.uint8)
        assert rows.shape == (self.n_layers, self.n_req, self.R)
        n = self.n_req if req_ids is None else len(req_ids)
        req = self._req(req_ids, n)
        status = np.zeros(n, dtype=np.int32)
        lib().orc_append(self.src, n, _p(req), _p(rows), _p(status), self.threads)
        return status

    def resolve(self, sel: np.ndarray, count=None, fill_layer: int = 0, req_ids=None):
        """sel: int32 [n][stride].  Returns loc, fills [n][B][2], fill_count, status."""
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        n, stride = sel.shape
        req = self._req(req_ids, n)
        cnt = None if count is None else np.ascontiguousarray(count, dtype=np.int32)
        loc = np.full((n, stride), INVALID, dtype=np.uint32)
        fills = np.full((n, self.B, 2), -1, dtype=np.int32)
        fill_count = np.zeros(n, dtype=np.int32)
        status = np.zeros(n, dtype=np.int32)
        stats = np.zeros(len(STAT_NAMES), dtype=np.uint64)
        lib().orc_resolve(self.src, n, _p(req), _p(sel), _p(cnt), stride, fill_layer, _p(loc),
                          _p(fills), _p(fill_count), _p(status), _p(stats), self.threads)
        self.stats += stats
        return loc, fills, fill_count, status

    def replay(self, layer: int, fills: np.ndarray, fill_count: np.ndarray, req_ids=None):
        fills = np.ascontiguousarray(fills, dtype=np.int32)
        fill_count = np.ascontiguousarray(fill_count, dtype=np.int32)
        n = fill_count.shape[0]
        assert fills.shape == (n, self.B, 2)
        req = self._req(req_ids, n)
        status = np.zeros(n, dtype=np.int32)
        lib().orc_replay(self.src, layer, n, _p(req), _p(fills), _p(fill_count), _p(status),
                         self.threads)
        return status

    def gather(self, layer: int, loc: np.ndarray, count=None, out=None, req_ids=None):
        """Returns (out uint8 [n][stride][R], status)."""
        loc = np.ascontiguousarray(loc, dtype=np.uint32)
        n, stride = loc.shape
        req = self._req(req_ids, n)
        cnt = None if count is None else np.ascontiguousarray(count, dtype=np.int32)
        if out is None:
            out = np.full((n, stride, self.R), 0xEE, dtype=np.uint8)
        assert out.shape == (n, stride, self.R) and out.flags.c_contiguous
        status = np.zeros(n, dtype=np.int32)
        lib().orc_gather(self.src, layer, n, _p(req), _p(loc), _p(cnt), stride, _p(out),
                         _p(status), self.threads)
        return out, status

    def dedup(self, sel: np.ndarray):
        """sel: int32 [n][q][k] -> union [n][q*k], union_count [n], map [n][q][k]."""
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        n, q, k = sel.shape
        union = np.full((n, q * k), -1, dtype=np.int32)
        ucount = np.zeros(n, dtype=np.int32)
        mp = np.full((n, q, k), -1, dtype=np.int32)
        lib().orc_dedup(self.src, n, q, k, _p(sel), _p(union), _p(ucount), _p(mp), self.threads)
        return union, ucount, mp

    def reclaim_pages(self, req, page):
        """Release the listed optional pages (backing up those without a host
        copy).  Returns (freed physical page or -1, status) per entry."""
        req = np.ascontiguousarray(req, dtype=np.int32)
        page = np.ascontiguousarray(page, dtype=np.int32)
        n = len(req)
        assert page.shape == (n,)
        freed = np.full(n, -1, dtype=np.int32)
        status = np.zeros(n, dtype=np.int32)
        lib().orc_reclaim_pages(self.src, n, _p(req), _p(page), _p(freed), _p(status))
        return freed, status

    def restore_pages(self, req, page, phys):
        """Make the listed pages ready in the given physical pages.  Returns
        the status per entry."""
        req = np.ascontiguousarray(req, dtype=np.int32)
        page = np.ascontiguousarray(page, dtype=np.int32)
        phys = np.ascontiguousarray(phys, dtype=np.int32)
        n = len(req)
        assert page.shape == (n,) and phys.shape == (n,)
        status = np.zeros(n, dtype=np.int32)
        lib().orc_restore_pages(self.src, n, _p(req), _p(page), _p(phys), _p(status))
        return status

    def check(self) -> np.ndarray:
        """Per request bit mask of violated state invariants (0 = all hold)."""
        return np.array([lib().orc_check_one(self.src, r) for r in range(self.n_req)],
                        dtype=np.int32)

    def snapshot(self) -> dict:
        return {"L": self.L.copy(), "tag": self.tag.copy(), "stamp": self.stamp.copy(),
                "clock": self.clock.copy(), "hot": [h.copy() for h in self.hot],
                "tail": [t.copy() for t in self.tail]}
