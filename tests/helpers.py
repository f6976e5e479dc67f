"""Small-input builders shared by the CPU tests (inputs only, no resolver rules)."""
from __future__ import annotations

import numpy as np

from oracle.oracle import OracleSource
from synth.gen import POISON_HOST, payload_np


def one_request_source(H, P, T, B, page_map, host_valid, R=32, n_layers=1, max_new=16, seed=7):
    """A single-request KV source with closed-form payload in every place."""
    n_pages = -(-H // P)
    page_map = np.asarray(page_map, dtype=np.int32).reshape(1, n_pages)
    host_valid = np.asarray(host_valid, dtype=np.uint8).reshape(1, n_pages)
    pool_pages = int(page_map.max()) + 1 if (page_map >= 0).any() else 0
    tail, pool, host = [], [], []
    for l in range(n_layers):
        t = np.full((1, T, R), POISON_HOST, dtype=np.uint8)
        for pos in range(max(0, H - T), H):
            t[0, pos % T] = payload_np(l, 0, pos, R, seed)
        p = np.zeros((pool_pages, P, R), dtype=np.uint8)
        for pg in range(n_pages):
            ph = page_map[0, pg]
            if ph >= 0:
                p[ph] = payload_np(l, 0, np.arange(pg * P, pg * P + P), R, seed)
        h = np.full((1, H + max_new, R), POISON_HOST, dtype=np.uint8)
        for pos in range(H):
            if host_valid[0, pos // P]:
                h[0, pos] = payload_np(l, 0, pos, R, seed)
        tail.append(t), pool.append(p), host.append(h)
    return OracleSource(n_req=1, n_layers=n_layers, H=H, max_new=max_new, P=P, T=T, B=B, R=R,
                        page_map=page_map, host_valid=host_valid, tail=tail, pool=pool,
                        host=host, threads=1)


def new_row(src: OracleSource, step_pos: int, seed=7) -> np.ndarray:
    """Payload of decoded position step_pos for every layer: [n_layers][1][R]."""
    return np.stack([payload_np(l, 0, step_pos, src.R, seed)[None] for l in range(src.n_layers)])
