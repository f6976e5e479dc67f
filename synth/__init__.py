"""Seeded synthetic workloads for the sparse KV row resolver (inputs only)."""
from .configs import FULL, REUSE_DISTINCT, REUSE_SHARED, Workload, tiny  # noqa: F401
from .gen import (POISON_FREE_PAGE, POISON_HOST, POISON_HOT, POISON_OUT, Inputs, build_lib,  # noqa: F401
                  payload_np)
