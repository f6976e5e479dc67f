"""Write tests/golden/*.json from the CPU oracle only.

Each fixture stores its own inputs (shape, page map, host-copy map, the
selection of every call) and the oracle's outputs, so it does not depend on
the input generator.  Run from the repository root:
    python tests/golden/make_golden.py
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle.oracle import OracleSource  # noqa: E402


def source(fx):
    n_pages = -(-fx["H"] // fx["P"])
    R, L = fx["R"], fx["n_layers"]
    zeros = lambda *s: np.zeros(s, dtype=np.uint8)  # noqa: E731
    pool_pages = max(fx["page_map"]) + 1 if max(fx["page_map"]) >= 0 else 0
    return OracleSource(n_req=1, n_layers=L, H=fx["H"], max_new=fx["max_new"], P=fx["P"],
                        T=fx["T"], B=fx["B"], R=R, page_map=np.array(fx["page_map"]),
                        host_valid=np.array(fx["host_valid"]),
                        tail=[zeros(1, fx["T"], R) for _ in range(L)],
                        pool=[zeros(pool_pages, fx["P"], R) for _ in range(L)],
                        host=[zeros(1, fx["H"] + fx["max_new"], R) for _ in range(L)], threads=1)


def run(fx):
    src = source(fx)
    out = []
    for call in fx["calls"]:
        if call.get("append"):
            src.append(np.zeros((fx["n_layers"], 1, fx["R"]), dtype=np.uint8))
        sel = np.array([call["sel"]], dtype=np.int32)
        loc, fills, fc, st = src.resolve(sel, fill_layer=0)
        out.append({"status": int(st[0]), "loc": [int(x) for x in loc[0]],
                    "fills": fills[0, : fc[0]].tolist(), "tag": src.tag[0].tolist(),
                    "stamp": [int(x) for x in src.stamp[0]], "clock": int(src.clock[0]),
                    "L": int(src.L[0])})
    return out


def scenario():
    rng = np.random.default_rng(2024)
    H, P, T, B = 96, 8, 6, 5
    page_map = [-1] * 12
    for i, pg in enumerate([0, 3, 4, 9]):
        page_map[pg] = 7 - i
    host_valid = [0 if p >= 0 else 1 for p in page_map]
    calls = []
    L = H
    for c in range(24):
        app = c % 3 == 1
        L += app
        sel = rng.choice(L, size=int(rng.integers(3, 9)), replace=False).tolist()
        calls.append({"append": app, "sel": sel})
    return {"name": "lru_trace_small", "H": H, "P": P, "T": T, "B": B, "R": 16, "n_layers": 1,
            "max_new": 12, "page_map": page_map, "host_valid": host_valid, "calls": calls,
            "note": "regression fixture written by tests/golden/make_golden.py from the oracle"}


if __name__ == "__main__":
    fx = scenario()
    fx["expected"] = run(fx)
    with open(os.path.join(HERE, fx["name"] + ".json"), "w") as f:
        json.dump(fx, f, indent=1)
    print("wrote", fx["name"])
