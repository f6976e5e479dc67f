"""The C ABI library loads and exports every call its header declares; host-side
argument checks work without a GPU (no compute call is made here)."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

from hierarchical_sparse_kv_resolve_amd import kvr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    text = open(os.path.join(ROOT, "include", "kvr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls_and_lifecycle():
    names = declared()
    for n in ("kvr_resolve_rows", "kvr_gather_rows", "kvr_dedup_verify_selections",
              "kvr_reuse_locations", "kvr_append_rows", "kvr_create", "kvr_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kvr.LIB_PATH)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing
    assert sorted(kvr.EXPORTS) == declared()


@pytest.mark.parametrize("field,value,msg", [
    ("hot_slots", 0, "hot_slots"), ("hot_slots", 8193, "hot_slots"),
    ("row_bytes", 24, "row_bytes"), ("sel_cap", 0, "sel_cap"), ("page_rows", 0, "page_rows"),
    ("pool_pages", 1 << 30, "pool_pages"), ("n_req", 0, "n_req"), ("tail_rows", -1, "tail_rows"),
])
def test_create_rejects_bad_shapes(field, value, msg):
    good = dict(n_req=2, n_layers=1, history_rows=100, max_new_rows=4, page_rows=8, tail_rows=4,
                hot_slots=16, row_bytes=32, sel_cap=16, pool_pages=3)
    good[field] = value
    with pytest.raises(kvr.KvrError) as e:
        kvr.Context(**good)
    assert e.value.code == kvr.E_ARG and msg in str(e.value)


def test_null_context_and_status_summary():
    lib = kvr.lib()
    assert lib.kvr_resolve_rows(None, 0, None, None, None, 0, None, None, None, -1, None, None,
                                None) == kvr.E_ARG
    assert "null context" in kvr.last_error()
    assert kvr.status_summary(np.array([0, 0, -2, 0, -3], dtype=np.int32)) == (2, 2)
    assert kvr.status_summary(np.zeros(3, dtype=np.int32)) == (0, -1)
    assert lib.kvr_destroy(None) == kvr.OK


def test_hot_path_calls_reject_a_null_context():
    lib = kvr.lib()
    layers = (ctypes.c_int32 * 1)(0)
    outs = (ctypes.c_void_p * 1)(None)
    assert lib.kvr_append_resolve_rows(None, 0, None, None, None, None, None, 0, None, None, None,
                                       -1, None, None, None) == kvr.E_ARG
    assert lib.kvr_append_rows(None, 0, None, None, None, None) == kvr.E_ARG
    for name in ("kvr_gather_rows", "kvr_gather_resident_rows"):
        assert getattr(lib, name)(None, 1, layers, 0, None, None, None, 0, outs, None,
                                  None) == kvr.E_ARG
    for name in ("kvr_fill_gather_rows", "kvr_fused_gather_rows"):
        assert getattr(lib, name)(None, 1, layers, 0, None, None, None, None, 0, outs, None,
                                  None) == kvr.E_ARG
        assert "null context" in kvr.last_error()


def test_deferred_and_combined_calls_reject_bad_arguments_on_the_host():
    """The deferred-append pair and the combined gather-resolve call refuse a
    null context, and the combined call refuses being given neither half,
    before any device work."""
    lib = kvr.lib()
    layers = (ctypes.c_int32 * 1)(0)
    outs = (ctypes.c_void_p * 1)(None)
    assert lib.kvr_append_resolve_rows_deferred(None, 0, None, None, None, None, None, None, 0,
                                                None, None, None, -1, None, None,
                                                None) == kvr.E_ARG
    assert "null context" in kvr.last_error()
    assert lib.kvr_fused_gather_append_rows(None, 1, layers, 0, None, None, None, None, 0, outs,
                                            None, None, None, None) == kvr.E_ARG
    assert "null context" in kvr.last_error()
    assert lib.kvr_gather_resolve_rows(None, None, None, None) == kvr.E_ARG
    assert "gather or a resolve" in kvr.last_error()
    g = kvr.GatherCall(1, ctypes.addressof(layers), 0, None, None, None, None, 0,
                       ctypes.addressof(outs), None, None, None)
    assert lib.kvr_gather_resolve_rows(None, ctypes.byref(g), None, None) == kvr.E_ARG
    assert "null context" in kvr.last_error()
    r = kvr.ResolveCall(0, None, None, None, None, None, None, 0, None, None, None, None, None)
    assert lib.kvr_gather_resolve_rows(None, None, ctypes.byref(r), None) == kvr.E_ARG
    assert "null context" in kvr.last_error()


def test_call_structs_match_the_header():
    """The binding's ctypes mirrors of kvr_gather_call and kvr_resolve_call
    have the header's field names in the header's order."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "kvr.h")).read(),
                  flags=re.S)
    for struct, cls in (("kvr_gather_call", kvr.GatherCall), ("kvr_resolve_call", kvr.ResolveCall)):
        body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (struct, struct), text, re.S).group(1)
        fields = re.findall(r"(\w+);", body)
        assert fields == [name for name, _ in cls._fields_], struct


def test_kernel_kinds_match_the_binding():
    text = open(os.path.join(ROOT, "include", "kvr.h")).read()
    kinds = {name.lower(): int(v) for name, v in re.findall(r"KVR_KERNEL_([A-Z]+)\s*=\s*(\d+)", text)}
    assert kinds == {name: i for i, name in enumerate(kvr.KERNEL_NAMES)}


def test_timing_calls_reject_a_null_context():
    lib = kvr.lib()
    assert lib.kvr_timing_begin(None, 8) == kvr.E_ARG
    assert lib.kvr_timing_end(None, 0, None, None, None) == kvr.E_ARG


def test_speculative_state_rejects_bad_shapes():
    lib = kvr.lib()
    out = ctypes.c_void_p()
    # window 0; capacity below the window; rows not a multiple of 16
    for args in ((2, 0, 4, 64), (2, 5, 4, 64), (2, 4, 8, 24)):
        assert lib.kvr_draft_create(*args, 1, 1, 1, ctypes.byref(out)) == kvr.E_ARG
    assert lib.kvr_draft_append(None, 0, None, 0, None, None, None) == kvr.E_ARG
    assert lib.kvr_staging_create(0, ctypes.byref(out)) == kvr.E_ARG
    assert lib.kvr_staging_acquire(None, None, None) == kvr.E_ARG
    assert lib.kvr_staging_release(None, 0, None) == kvr.E_ARG


def test_binding_argument_checks_on_the_host():
    """The binding's own checks that need no GPU: host tensors and arrays are
    refused as device arguments, unpinned tensors as the host store, and plain
    addresses and NULL pass through unchanged."""
    import torch
    with pytest.raises(TypeError, match="expected a GPU tensor"):
        kvr._dev(torch.zeros(4), "sel")
    with pytest.raises(TypeError, match="or an address"):
        kvr._dev(np.zeros(4), "sel")
    with pytest.raises(TypeError, match="pinned host tensor"):
        kvr._pinned(torch.zeros(4), "host")
    assert kvr._dev(None, "status") is None
    assert kvr._dev(4096, "sel", 1 << 40) == 4096
    assert kvr._pinned(8192, "host", 1 << 40) == 8192
