"""Workload shapes for the per-decode-step sparse KV row resolver.

Five serving shapes follow the evaluation settings of "Adaptive DHiSparse:
Speculative Decoding over a Load-Adaptive KV Hierarchy" (How it works,
Evidence): GLM-style 32K-row histories at C8/C64, a speculative verify block,
and a DeepSeek-style 524288-row context whose Reuse layers inherit a location
vector.  The tiny shapes exist so that the CPU reference finishes in well under
a second while still spanning several kernel tiles and ragged tails.

This module holds only shapes and knobs; it performs none of the resolver's
arithmetic.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

# How a step's model layers obtain their payload:
#   "distinct": every payload layer shares the one location vector, and the
#               rows filled for layer 0 are replayed from each other layer's
#               host store (GLM-style shared sparse indices).
#   "shared":   one physical payload layer; layers after a resolving layer
#               inherit its location vector and gathered buffer (DeepSeek-style).
REUSE_DISTINCT = "distinct"
REUSE_SHARED = "shared"


@dataclass(frozen=True)
class Workload:
    name: str
    n_req: int            # concurrent requests
    H: int                # imported history rows per request
    R: int                # row bytes
    P: int                # page size in rows
    T: int                # tail rows
    ready_frac: float     # fraction of complete imported pages that are ready on device
    B: int                # hot-cache slots per (request, KV source)
    k: int                # top-k selected rows per query
    steps: int            # decode steps
    payload_layers: int = 1      # distinct payload layers of the one KV source
    groups: int = 1              # resolving layers per step (each with its own selection)
    layers_per_group: int = 1    # model layers served by one resolving layer
    reuse: str = REUSE_DISTINCT
    q: int = 1                   # verification queries per request (1 = no verify block)
    shared_frac: float = 0.0     # share of query 0's rows reused by queries 1..q-1
    sel: str = "uniform"         # "mix", "zipf" or "uniform"
    zipf_s: float = 0.0
    mix_recent: int = 0          # "mix": window of most recent rows
    mix_recent_frac: float = 0.0  # "mix": share of k drawn from that window
    seed: int = 0
    pool_spare: int = 0          # optional-pool pages no request holds at admission

    @property
    def n_pages(self) -> int:
        """Page-map entries per request: one per started page of history."""
        return -(-self.H // self.P)

    @property
    def full_pages(self) -> int:
        return self.H // self.P

    @property
    def ready_pages(self) -> int:
        """Ready pages per request: the fraction of complete pages, rounded."""
        return int(round(self.ready_frac * self.full_pages))

    @property
    def pool_pages(self) -> int:
        return self.ready_pages * self.n_req + self.pool_spare

    @property
    def sel_cap(self) -> int:
        """Selection capacity of one resolve call (the union capacity for verify)."""
        return self.q * self.k

    @property
    def model_layers(self) -> int:
        if self.reuse == REUSE_SHARED:
            return self.groups * self.layers_per_group
        return self.payload_layers

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Full-size shapes.  Unstated knobs take the plainest reading:
#  * memory-pressure and verify shapes reuse the 256-row tail of the other
#    32K-history shape, and the verify shape reuses its page size, Zipf
#    exponent and ready fraction;
#  * the long-context shape uses one physical payload source for all 12 layers
#    (4 resolving layers, each followed by 2 Reuse layers).
C1 = Workload(name="c1_single_request", n_req=1, H=4096, R=1152, P=64, T=128,
              ready_frac=0.5, B=512, k=256, steps=8, sel="mix", mix_recent=1024,
              mix_recent_frac=0.7, seed=1001)
C2 = Workload(name="c2_glm_shared_indices", n_req=8, H=32768, R=1152, P=64, T=256,
              ready_frac=0.7, B=4096, k=2048, steps=32, payload_layers=8,
              sel="zipf", zipf_s=1.1, seed=1002)
C3 = Workload(name="c3_memory_pressure", n_req=64, H=32768, R=1152, P=64, T=256,
              ready_frac=0.1, B=2048, k=2048, steps=16, sel="uniform", seed=1003)
C4 = Workload(name="c4_speculative_verify", n_req=32, H=32768, R=1152, P=64, T=256,
              ready_frac=0.7, B=4096, k=2048, steps=16, payload_layers=4, q=4,
              shared_frac=0.8, sel="zipf", zipf_s=1.1, seed=1004)
C5 = Workload(name="c5_deepseek_long_context", n_req=64, H=524288, R=656, P=64, T=512,
              ready_frac=0.3, B=8192, k=2048, steps=8, payload_layers=1, groups=4,
              layers_per_group=3, reuse=REUSE_SHARED, sel="zipf", zipf_s=1.05,
              seed=1005)

FULL = {1: C1, 2: C2, 3: C3, 4: C4, 5: C5}


def tiny(c: int) -> Workload:
    """A reduced copy of shape c that the CPU reference runs in well under a second.

    Sizes keep several 64-lane tiles, ragged row counts (not multiples of 64)
    and real eviction pressure (B below the number of distinct pending rows).
    """
    base = FULL[c]
    if c == 1:
        return base.with_(name="t1", H=700, T=40, B=96, k=75, steps=6, mix_recent=200)
    if c == 2:
        return base.with_(name="t2", n_req=3, H=1500, T=37, B=100, k=90, steps=7,
                          payload_layers=3)
    if c == 3:
        return base.with_(name="t3", n_req=5, H=1300, T=33, B=180, k=180, steps=5)
    if c == 4:
        return base.with_(name="t4", n_req=3, H=1400, T=31, B=300, k=90, steps=5,
                          payload_layers=2)
    if c == 5:
        return base.with_(name="t5", n_req=4, H=6000, R=656, T=45, B=260, k=100,
                          steps=4, groups=3)
    raise ValueError(c)
