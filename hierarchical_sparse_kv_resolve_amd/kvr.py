"""Thin ctypes binding of libkvr.so (include/kvr.h).

Argument marshalling only: every entry point forwards raw device pointers,
sizes and a HIP stream to the C ABI, and raises KvrError on a non-OK return.
All work on the path runs in the library's HIP kernels; there is no fallback.
Tensors may be torch tensors (their data_ptr() is passed), plain integer
addresses, or None for NULL.  A torch tensor is checked against what the
header says of its argument (on the GPU or pinned host memory, contiguous, at
least the bytes the call reads or writes) before the call; addresses are
passed as given.  The stream defaults to torch's current stream.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvr.so")

OK = 0
E_ARG = -1
E_RANGE = -2
E_CAPACITY = -3
E_NO_HOST_COPY = -4
E_HIP = -5
E_STATE = -6

PLACE_TAIL, PLACE_PAGE, PLACE_HOT, PLACE_INVALID = 0, 1, 2, 3
LOC_INVALID = 0xFFFFFFFF
REUSE_SHARED_SOURCE = 0
REUSE_DISTINCT_PAYLOAD = 1

# Every entry point of include/kvr.h.
EXPORTS = ("kvr_create", "kvr_destroy", "kvr_last_error", "kvr_bind_metadata", "kvr_bind_layer",
           "kvr_init_state", "kvr_append_rows", "kvr_resolve_rows", "kvr_append_resolve_rows",
           "kvr_append_resolve_rows_deferred", "kvr_gather_rows", "kvr_fused_gather_append_rows",
           "kvr_gather_resolve_rows",
           "kvr_dedup_verify_selections", "kvr_reuse_locations", "kvr_status_summary",
           "kvr_host_alloc", "kvr_host_free", "kvr_timing_begin", "kvr_timing_end",
           "kvr_reclaim_pages", "kvr_restore_pages", "kvr_gather_resident_rows",
           "kvr_fill_gather_rows", "kvr_fused_gather_rows", "kvr_residency_create",
           "kvr_residency_destroy", "kvr_residency_admit", "kvr_residency_release",
           "kvr_residency_refill", "kvr_residency_counts", "kvr_draft_create",
           "kvr_draft_destroy", "kvr_draft_reset", "kvr_draft_append", "kvr_draft_rollback",
           "kvr_draft_window", "kvr_staging_create", "kvr_staging_destroy",
           "kvr_staging_acquire", "kvr_staging_release")

# kvr_kernel: kinds of the library's kernel launches (launch timing).
KERNEL_NAMES = ("append", "resolve", "refill", "gather", "dedup", "state", "fused", "step")


class KvrError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"kvr error {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("history_rows", ctypes.c_int32), ("max_new_rows", ctypes.c_int32),
                ("page_rows", ctypes.c_int32), ("tail_rows", ctypes.c_int32),
                ("hot_slots", ctypes.c_int32), ("row_bytes", ctypes.c_int32),
                ("sel_cap", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("pool_pages", ctypes.c_int64)]


STATS_FIELDS = ("calls", "tail", "page", "hit", "miss", "fill", "host_bytes", "error")


class GatherCall(ctypes.Structure):
    """kvr_gather_call of include/kvr.h."""
    _fields_ = [("n_layers", ctypes.c_int32), ("layers", ctypes.c_void_p),
                ("n", ctypes.c_int32), ("req_ids", ctypes.c_void_p), ("loc", ctypes.c_void_p),
                ("sel", ctypes.c_void_p), ("count", ctypes.c_void_p), ("stride", ctypes.c_int32),
                ("out", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("new_rows", ctypes.c_void_p), ("append_pos", ctypes.c_void_p)]


class ResolveCall(ctypes.Structure):
    """kvr_resolve_call of include/kvr.h."""
    _fields_ = [("n", ctypes.c_int32), ("req_ids", ctypes.c_void_p),
                ("new_rows", ctypes.c_void_p), ("append_status", ctypes.c_void_p),
                ("append_pos", ctypes.c_void_p), ("sel", ctypes.c_void_p),
                ("sel_count", ctypes.c_void_p), ("stride", ctypes.c_int32),
                ("loc", ctypes.c_void_p), ("fills", ctypes.c_void_p),
                ("fill_count", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("stats", ctypes.c_void_p)]

_lib = None


def lib():
    """Load libkvr.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m hierarchical_sparse_kv_resolve_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, U = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sig = {
            "kvr_create": [P, P],
            "kvr_destroy": [P],
            "kvr_bind_metadata": [P, P, P, P, P, P, P],
            "kvr_bind_layer": [P, I, P, P, P, P],
            "kvr_init_state": [P, P],
            "kvr_append_rows": [P, I, P, P, P, P],
            "kvr_resolve_rows": [P, I, P, P, P, I, P, P, P, I, P, P, P],
            "kvr_append_resolve_rows": [P, I, P, P, P, P, P, I, P, P, P, I, P, P, P],
            "kvr_append_resolve_rows_deferred": [P, I, P, P, P, P, P, P, I, P, P, P, I, P, P, P],
            "kvr_gather_rows": [P, I, P, I, P, P, P, I, P, P, P],
            "kvr_gather_resident_rows": [P, I, P, I, P, P, P, I, P, P, P],
            "kvr_fill_gather_rows": [P, I, P, I, P, P, P, P, I, P, P, P],
            "kvr_fused_gather_rows": [P, I, P, I, P, P, P, P, I, P, P, P],
            "kvr_fused_gather_append_rows": [P, I, P, I, P, P, P, P, I, P, P, P, P, P],
            "kvr_gather_resolve_rows": [P, P, P, P],
            "kvr_dedup_verify_selections": [P, I, I, I, P, P, P, P, P],
            "kvr_reuse_locations": [P, I, I, P, I, P, P, P, P, I, P, P, P, P],
            "kvr_status_summary": [P, I, P],
            "kvr_host_alloc": [U, P],
            "kvr_host_free": [P],
            "kvr_timing_begin": [P, I],
            "kvr_timing_end": [P, I, P, P, P],
            "kvr_reclaim_pages": [P, I, P, P, P, P, P],
            "kvr_restore_pages": [P, I, P, P, P, P, P],
            "kvr_residency_create": [I, I, I, ctypes.c_int64, P, P],
            "kvr_residency_destroy": [P],
            "kvr_residency_admit": [P, ctypes.c_int64, I, P, I, P, P, P, P],
            "kvr_residency_release": [P, I],
            "kvr_residency_refill": [P, I, I, P, P, P, P],
            "kvr_residency_counts": [P, P, P, P],
            "kvr_draft_create": [I, I, I, I, P, P, P, P],
            "kvr_draft_destroy": [P],
            "kvr_draft_reset": [P, P],
            "kvr_draft_append": [P, I, P, I, P, P, P],
            "kvr_draft_rollback": [P, I, P, P, P, P],
            "kvr_draft_window": [P, I, P, P, P, P, P],
            "kvr_staging_create": [I, P],
            "kvr_staging_destroy": [P],
            "kvr_staging_acquire": [P, P, P],
            "kvr_staging_release": [P, I, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.kvr_last_error.argtypes = []
        L.kvr_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):  # numpy array (host memory)
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _dev(x, name: str, nbytes: int = 0) -> int | None:
    """Address of a device argument.  A torch tensor must live on the GPU, be
    contiguous and hold at least `nbytes` (the size the header's layout gives
    it for this call), so that a host tensor or a short buffer raises here
    instead of reaching a kernel.  Integer addresses and None pass unchecked."""
    if x is None or isinstance(x, int):
        return x
    if hasattr(x, "is_cuda"):
        if not x.is_cuda:
            raise TypeError(f"{name}: expected a GPU tensor, got one on {x.device}")
        if not x.is_contiguous():
            raise ValueError(f"{name}: the tensor is not contiguous")
        have = x.numel() * x.element_size()
        if have < nbytes:
            raise ValueError(f"{name}: {have} bytes, the call needs {nbytes}")
        return x.data_ptr()
    raise TypeError(f"{name}: expected a GPU tensor or an address, got {type(x)}")


def _pinned(x, name: str, nbytes: int = 0) -> int | None:
    """Address of a pinned host argument (a torch tensor in pinned CPU memory,
    or an address from host_alloc)."""
    if x is None or isinstance(x, int):
        return x
    if hasattr(x, "is_cuda"):
        if x.is_cuda or not x.is_pinned():
            raise TypeError(f"{name}: expected a pinned host tensor")
        if not x.is_contiguous():
            raise ValueError(f"{name}: the tensor is not contiguous")
        have = x.numel() * x.element_size()
        if have < nbytes:
            raise ValueError(f"{name}: {have} bytes, the call needs {nbytes}")
        return x.data_ptr()
    raise TypeError(f"{name}: expected a pinned host tensor or an address, got {type(x)}")


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc != OK:
        raise KvrError(rc, lib().kvr_last_error().decode())
    return rc


def last_error() -> str:
    return lib().kvr_last_error().decode()


def host_alloc(nbytes: int) -> int:
    out = ctypes.c_void_p()
    _check(lib().kvr_host_alloc(nbytes, ctypes.byref(out)))
    return out.value


def host_free(ptr: int) -> None:
    _check(lib().kvr_host_free(ptr))


def status_summary(status_host) -> tuple[int, int]:
    """(number of failed requests, index of the first or -1) of a host int32 array."""
    import numpy as np
    st = np.ascontiguousarray(status_host, dtype=np.int32)
    first = ctypes.c_int32()
    bad = lib().kvr_status_summary(st.ctypes.data, len(st), ctypes.byref(first))
    if bad < 0:
        _check(bad)
    return bad, first.value


class Context:
    """One KV source: n_req requests and n_layers payload layers."""

    def __init__(self, *, n_req, n_layers, history_rows, max_new_rows, page_rows, tail_rows,
                 hot_slots, row_bytes, sel_cap, pool_pages):
        self.cfg = Config(n_req, n_layers, history_rows, max_new_rows, page_rows, tail_rows,
                          hot_slots, row_bytes, sel_cap, 0, pool_pages)
        h = ctypes.c_void_p()
        _check(lib().kvr_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self.handle = h.value
        self._keep = []

    def close(self):
        if self.handle:
            lib().kvr_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _sizes(self):
        c = self.cfg
        return (c.n_req, c.n_layers, c.history_rows, c.max_new_rows, c.page_rows, c.tail_rows,
                c.hot_slots, c.row_bytes, c.pool_pages)

    def bind_metadata(self, L, page_map, host_valid, tag, stamp, clock):
        N, _, H, _, P, _, B, _, _ = self._sizes()
        npg = (H + P - 1) // P if P > 0 else 0
        _check(lib().kvr_bind_metadata(self.handle, _dev(L, "L", 4 * N),
                                       _dev(page_map, "page_map", 4 * N * npg),
                                       _dev(host_valid, "host_valid", N * npg),
                                       _dev(tag, "tag", 4 * N * B), _dev(stamp, "stamp", 4 * N * B),
                                       _dev(clock, "clock", 4 * N)))

    def bind_layer(self, layer, tail, pool, hot, host):
        N, _, H, M, P, T, B, R, pool_pages = self._sizes()
        _check(lib().kvr_bind_layer(self.handle, layer, _dev(tail, "tail", N * T * R),
                                    _dev(pool, "pool", pool_pages * P * R),
                                    _dev(hot, "hot", N * B * R),
                                    _pinned(host, "host", N * (H + M) * R)))

    def init_state(self, stream=None):
        _check(lib().kvr_init_state(self.handle, _stream(stream)))

    def append_rows(self, n, req_ids, new_rows, status=None, stream=None):
        _, NL, _, _, _, _, _, R, _ = self._sizes()
        _check(lib().kvr_append_rows(self.handle, n, _dev(req_ids, "req_ids", 4 * n),
                                     _dev(new_rows, "new_rows", NL * n * R),
                                     _dev(status, "status", 4 * n), _stream(stream)))

    def _resolve_args(self, n, req_ids, sel, sel_count, stride, loc, fills, fill_count, status,
                      stats):
        B = self.cfg.hot_slots
        m = max(n, 0) * max(stride, 0)
        return (_dev(req_ids, "req_ids", 4 * n), _dev(sel, "sel", 4 * m),
                _dev(sel_count, "sel_count", 4 * n), _dev(loc, "loc", 4 * m),
                _dev(fills, "fills", 8 * n * B), _dev(fill_count, "fill_count", 4 * n),
                _dev(status, "status", 4 * n), _dev(stats, "stats", 8 * len(STATS_FIELDS)))

    def resolve_rows(self, n, req_ids, sel, sel_count, stride, loc, fills, fill_count, fill_layer,
                     status, stats=None, stream=None):
        rid, sl, sc, lc, fl, fc, st, sts = self._resolve_args(n, req_ids, sel, sel_count, stride,
                                                              loc, fills, fill_count, status,
                                                              stats)
        _check(lib().kvr_resolve_rows(self.handle, n, rid, sl, sc, stride, lc, fl, fc, fill_layer,
                                      st, sts, _stream(stream)))

    def append_resolve_rows(self, n, req_ids, new_rows, append_status, sel, sel_count, stride, loc,
                            fills, fill_count, fill_layer, status, stats=None, stream=None):
        NL, R = self.cfg.n_layers, self.cfg.row_bytes
        rid, sl, sc, lc, fl, fc, st, sts = self._resolve_args(n, req_ids, sel, sel_count, stride,
                                                              loc, fills, fill_count, status,
                                                              stats)
        _check(lib().kvr_append_resolve_rows(self.handle, n, rid,
                                             _dev(new_rows, "new_rows", NL * n * R),
                                             _dev(append_status, "append_status", 4 * n), sl, sc,
                                             stride, lc, fl, fc, fill_layer, st, sts,
                                             _stream(stream)))

    def append_resolve_rows_deferred(self, n, req_ids, new_rows, append_status, append_pos, sel,
                                     sel_count, stride, loc, fills, fill_count, fill_layer,
                                     status, stats=None, stream=None):
        NL, R = self.cfg.n_layers, self.cfg.row_bytes
        rid, sl, sc, lc, fl, fc, st, sts = self._resolve_args(n, req_ids, sel, sel_count, stride,
                                                              loc, fills, fill_count, status,
                                                              stats)
        _check(lib().kvr_append_resolve_rows_deferred(
            self.handle, n, rid, _dev(new_rows, "new_rows", NL * n * R),
            _dev(append_status, "append_status", 4 * n), _dev(append_pos, "append_pos", 4 * n),
            sl, sc, stride, lc, fl, fc, fill_layer, st, sts, _stream(stream)))

    def _gather_args(self, layers, n, req_ids, loc, count, stride, outs, status):
        nl = len(layers)
        m = max(n, 0) * max(stride, 0)
        R = self.cfg.row_bytes
        if len(outs) != nl:
            raise ValueError(f"outs: {len(outs)} buffers for {nl} layers")
        arr_l = (ctypes.c_int32 * max(1, nl))(*layers)
        arr_o = (ctypes.c_void_p * max(1, nl))(*[_dev(o, "out", m * R) for o in outs])
        return (nl, arr_l, _dev(req_ids, "req_ids", 4 * n), _dev(loc, "loc", 4 * m),
                _dev(count, "count", 4 * n), arr_o, _dev(status, "status", 4 * n))

    def gather_rows(self, layers, n, req_ids, loc, count, stride, outs, status=None, stream=None):
        nl, arr_l, rid, lc, cnt, arr_o, st = self._gather_args(layers, n, req_ids, loc, count,
                                                               stride, outs, status)
        _check(lib().kvr_gather_rows(self.handle, nl, arr_l, n, rid, lc, cnt, stride, arr_o, st,
                                     _stream(stream)))

    def gather_resident_rows(self, layers, n, req_ids, loc, count, stride, outs, status=None,
                             stream=None):
        nl, arr_l, rid, lc, cnt, arr_o, st = self._gather_args(layers, n, req_ids, loc, count,
                                                               stride, outs, status)
        _check(lib().kvr_gather_resident_rows(self.handle, nl, arr_l, n, rid, lc, cnt, stride,
                                              arr_o, st, _stream(stream)))

    def fill_gather_rows(self, layers, n, req_ids, loc, sel, count, stride, outs, status=None,
                         stream=None):
        nl, arr_l, rid, lc, cnt, arr_o, st = self._gather_args(layers, n, req_ids, loc, count,
                                                               stride, outs, status)
        sl = _dev(sel, "sel", 4 * max(n, 0) * max(stride, 0))
        _check(lib().kvr_fill_gather_rows(self.handle, nl, arr_l, n, rid, lc, sl, cnt, stride,
                                          arr_o, st, _stream(stream)))

    def fused_gather_rows(self, layers, n, req_ids, loc, sel, count, stride, outs, status=None,
                          stream=None):
        nl, arr_l, rid, lc, cnt, arr_o, st = self._gather_args(layers, n, req_ids, loc, count,
                                                               stride, outs, status)
        sl = _dev(sel, "sel", 4 * max(n, 0) * max(stride, 0))
        _check(lib().kvr_fused_gather_rows(self.handle, nl, arr_l, n, rid, lc, sl, cnt, stride,
                                           arr_o, st, _stream(stream)))

    def fused_gather_append_rows(self, layers, n, req_ids, loc, sel, count, stride, outs,
                                 new_rows, append_pos, status=None, stream=None):
        nl, arr_l, rid, lc, cnt, arr_o, st = self._gather_args(layers, n, req_ids, loc, count,
                                                               stride, outs, status)
        sl = _dev(sel, "sel", 4 * max(n, 0) * max(stride, 0))
        NL, R = self.cfg.n_layers, self.cfg.row_bytes
        _check(lib().kvr_fused_gather_append_rows(
            self.handle, nl, arr_l, n, rid, lc, sl, cnt, stride, arr_o, st,
            _dev(new_rows, "new_rows", NL * n * R), _dev(append_pos, "append_pos", 4 * n),
            _stream(stream)))

    def gather_resolve_rows(self, gather=None, resolve=None, stream=None):
        """kvr_gather_resolve_rows.  gather: dict(layers, n, req_ids, loc, sel,
        count, stride, outs, status, new_rows, append_pos) or None; resolve:
        dict(n, req_ids, new_rows, append_status, append_pos, sel, sel_count,
        stride, loc, fills, fill_count, status, stats) or None.  Missing keys
        are NULL."""
        keep = []
        g_ptr = r_ptr = None
        NL, R = self.cfg.n_layers, self.cfg.row_bytes
        if gather is not None:
            g = {**dict(req_ids=None, count=None, status=None, new_rows=None, append_pos=None,
                        sel=None), **gather}
            n, stride = g["n"], g["stride"]
            nl, arr_l, rid, lc, cnt, arr_o, st = self._gather_args(
                g["layers"], n, g["req_ids"], g["loc"], g["count"], stride, g["outs"], g["status"])
            gc = GatherCall(nl, ctypes.addressof(arr_l), n, rid, lc,
                            _dev(g["sel"], "sel", 4 * max(n, 0) * max(stride, 0)), cnt, stride,
                            ctypes.addressof(arr_o), st,
                            _dev(g["new_rows"], "new_rows", NL * n * R),
                            _dev(g["append_pos"], "append_pos", 4 * n))
            keep += [arr_l, arr_o, gc]
            g_ptr = ctypes.addressof(gc)
        if resolve is not None:
            r = {**dict(req_ids=None, new_rows=None, append_status=None, append_pos=None,
                        sel_count=None, stats=None), **resolve}
            n = r["n"]
            rid, sl, sc, lc, fl, fc, st, sts = self._resolve_args(
                n, r["req_ids"], r["sel"], r["sel_count"], r["stride"], r["loc"], r["fills"],
                r["fill_count"], r["status"], r["stats"])
            rc = ResolveCall(n, rid, _dev(r["new_rows"], "new_rows", NL * n * R),
                             _dev(r["append_status"], "append_status", 4 * n),
                             _dev(r["append_pos"], "append_pos", 4 * n), sl, sc, r["stride"], lc,
                             fl, fc, st, sts)
            keep.append(rc)
            r_ptr = ctypes.addressof(rc)
        _check(lib().kvr_gather_resolve_rows(self.handle, g_ptr, r_ptr, _stream(stream)))

    def dedup_verify_selections(self, n, q, k, sel, union_rows, union_count, map_, stream=None):
        m = max(n, 0) * max(q, 0) * max(k, 0)
        _check(lib().kvr_dedup_verify_selections(self.handle, n, q, k, _dev(sel, "sel", 4 * m),
                                                 _dev(union_rows, "union_rows", 4 * m),
                                                 _dev(union_count, "union_count", 4 * n),
                                                 _dev(map_, "map", 4 * m), _stream(stream)))

    def timing_begin(self, capacity: int):
        """Record the duration of each kernel this context launches from now on
        (events on the launches themselves; measurement aid)."""
        _check(lib().kvr_timing_begin(self.handle, capacity))
        self._timing_cap = capacity

    def timing_end(self):
        """Stop recording; waits for the recorded launches.  Returns a list of
        (kernel name, milliseconds) in launch order."""
        import numpy as np
        cap = getattr(self, "_timing_cap", 0)
        kinds = np.zeros(max(1, cap), dtype=np.int32)
        ms = np.zeros(max(1, cap), dtype=np.float32)
        n = ctypes.c_int32()
        _check(lib().kvr_timing_end(self.handle, cap, kinds.ctypes.data, ms.ctypes.data,
                                    ctypes.byref(n)))
        m = min(n.value, cap)
        return [(KERNEL_NAMES[k], float(t)) for k, t in zip(kinds[:m], ms[:m])]

    def reclaim_pages(self, n, req_ids, pages, freed_phys, status=None, stream=None):
        _check(lib().kvr_reclaim_pages(self.handle, n, _dev(req_ids, "req_ids", 4 * n),
                                       _dev(pages, "pages", 4 * n),
                                       _dev(freed_phys, "freed_phys", 4 * n),
                                       _dev(status, "status", 4 * n), _stream(stream)))

    def restore_pages(self, n, req_ids, pages, phys, status=None, stream=None):
        _check(lib().kvr_restore_pages(self.handle, n, _dev(req_ids, "req_ids", 4 * n),
                                       _dev(pages, "pages", 4 * n), _dev(phys, "phys", 4 * n),
                                       _dev(status, "status", 4 * n), _stream(stream)))

    def reuse_locations(self, mode, dst_layers, n, req_ids, src_loc, dst_loc, count, stride,
                        fills=None, fill_count=None, status=None, stream=None):
        layers = list(dst_layers or [])
        arr_l = (ctypes.c_int32 * max(1, len(layers)))(*layers)
        m = max(n, 0) * max(stride, 0)
        B = self.cfg.hot_slots
        _check(lib().kvr_reuse_locations(self.handle, mode, len(layers), arr_l, n,
                                         _dev(req_ids, "req_ids", 4 * n),
                                         _dev(src_loc, "src_loc", 4 * m),
                                         _dev(dst_loc, "dst_loc", 4 * m),
                                         _dev(count, "count", 4 * n),
                                         stride, _dev(fills, "fills", 8 * n * B),
                                         _dev(fill_count, "fill_count", 4 * n),
                                         _dev(status, "status", 4 * n), _stream(stream)))


class Residency:
    """Host-side residency policy of one source's optional pool
    (kvr_residency_*): which pages to reclaim for an admission and which to
    refill.  Its decisions are applied with Context.reclaim_pages and
    Context.restore_pages."""

    def __init__(self, page_map, n_complete: int, pool_pages: int):
        import numpy as np
        pm = np.ascontiguousarray(page_map, dtype=np.int32)
        self.n_req, self.n_pages = pm.shape
        self.n_complete = int(n_complete)
        h = ctypes.c_void_p()
        _check(lib().kvr_residency_create(self.n_req, self.n_pages, self.n_complete,
                                          int(pool_pages), pm.ctypes.data, ctypes.byref(h)))
        self.handle = h.value

    def close(self):
        if self.handle:
            lib().kvr_residency_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def admit(self, need: int, order):
        """(True, [(request, page), ...] to reclaim, handle), or (False, [], -1)
        when the shortfall is larger than all optional pages together."""
        import numpy as np
        order = np.ascontiguousarray(order, dtype=np.int32)
        cap = self.n_req * self.n_complete
        req = np.zeros(max(1, cap), dtype=np.int32)
        page = np.zeros(max(1, cap), dtype=np.int32)
        n, h = ctypes.c_int32(), ctypes.c_int32()
        rc = lib().kvr_residency_admit(self.handle, int(need), len(order), order.ctypes.data, cap,
                                       req.ctypes.data, page.ctypes.data, ctypes.byref(n),
                                       ctypes.byref(h))
        if rc == E_CAPACITY:
            return False, [], -1
        _check(rc)
        return True, list(zip(req[:n.value].tolist(), page[:n.value].tolist())), h.value

    def release(self, handle: int):
        _check(lib().kvr_residency_release(self.handle, handle))

    def refill(self, bound: int):
        """[(request, page, physical page), ...] to restore."""
        import numpy as np
        cap = max(1, bound)
        req = np.zeros(cap, dtype=np.int32)
        page = np.zeros(cap, dtype=np.int32)
        phys = np.zeros(cap, dtype=np.int32)
        n = ctypes.c_int32()
        _check(lib().kvr_residency_refill(self.handle, bound, cap, req.ctypes.data,
                                          page.ctypes.data, phys.ctypes.data, ctypes.byref(n)))
        m = n.value
        return list(zip(req[:m].tolist(), page[:m].tolist(), phys[:m].tolist()))

    def counts(self):
        """(free pages, ready pages, reserved pages)."""
        f, r, s = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().kvr_residency_counts(self.handle, ctypes.byref(f), ctypes.byref(r),
                                          ctypes.byref(s)))
        return f.value, r.value, s.value


class DraftRing:
    """Drafter visible-window ring (kvr_draft_*) over caller-owned device
    buffers: ring [n_req][capacity][row_bytes], length and high int32 [n_req]."""

    def __init__(self, n_req, window, capacity, row_bytes, ring, length, high):
        h = ctypes.c_void_p()
        self.n_req, self.window_rows, self.row_bytes = n_req, window, row_bytes
        _check(lib().kvr_draft_create(n_req, window, capacity, row_bytes,
                                      _dev(ring, "ring", max(n_req, 0) * max(capacity, 0) *
                                           max(row_bytes, 0)),
                                      _dev(length, "length", 4 * max(n_req, 0)),
                                      _dev(high, "high", 4 * max(n_req, 0)), ctypes.byref(h)))
        self.handle = h.value

    def close(self):
        if self.handle:
            lib().kvr_draft_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self, stream=None):
        _check(lib().kvr_draft_reset(self.handle, _stream(stream)))

    def append(self, n, req_ids, rows_each, rows, status=None, stream=None):
        need = max(n, 0) * max(rows_each, 0) * self.row_bytes
        _check(lib().kvr_draft_append(self.handle, n, _dev(req_ids, "req_ids", 4 * n), rows_each,
                                      _dev(rows, "rows", need), _dev(status, "status", 4 * n),
                                      _stream(stream)))

    def rollback(self, n, req_ids, keep, status=None, stream=None):
        _check(lib().kvr_draft_rollback(self.handle, n, _dev(req_ids, "req_ids", 4 * n),
                                        _dev(keep, "keep", 4 * n), _dev(status, "status", 4 * n),
                                        _stream(stream)))

    def window(self, n, req_ids, out, visible=None, status=None, stream=None):
        need = max(n, 0) * self.window_rows * self.row_bytes
        _check(lib().kvr_draft_window(self.handle, n, _dev(req_ids, "req_ids", 4 * n),
                                      _dev(out, "out", need), _dev(visible, "visible", 4 * n),
                                      _dev(status, "status", 4 * n), _stream(stream)))


class StagingPool:
    """Verification staging reuse (kvr_staging_*): buffer indices handed out
    round-robin; acquire waits for the buffer's last release."""

    def __init__(self, n_buffers: int):
        h = ctypes.c_void_p()
        _check(lib().kvr_staging_create(n_buffers, ctypes.byref(h)))
        self.handle = h.value

    def close(self):
        if self.handle:
            lib().kvr_staging_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def acquire(self, stream=None) -> int:
        idx = ctypes.c_int32()
        _check(lib().kvr_staging_acquire(self.handle, _stream(stream), ctypes.byref(idx)))
        return idx.value

    def release(self, index: int, stream=None):
        _check(lib().kvr_staging_release(self.handle, index, _stream(stream)))
