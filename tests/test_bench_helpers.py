"""Host-side helpers of bench.py (CPU only): the recorded traffic is used only
for the workload, schedule and gather source it was measured on; launch
records group by kernel; layer groups split the payload layers."""
from __future__ import annotations

import os

import numpy as np
import pytest

import bench
from hierarchical_sparse_kv_resolve_amd.runner import layer_groups


def test_recorded_traffic_matches_workload_schedule_and_source():
    records = bench.traffic_records()
    assert records, "no counter summaries under profiles/"
    for fields in records:
        wl, sched = fields["workload"], fields["schedule"]
        kernel = fields.get("kernel", "gather_kernel")
        if fields["source_sha256"] == bench.gather_source_hash():
            assert bench.recorded_traffic(wl, sched, kernel) == int(
                fields["traffic_bytes_per_launch"])
        else:  # the gather source changed since the counters were taken
            assert bench.recorded_traffic(wl, sched, kernel) is None
        assert bench.recorded_traffic(wl, sched, "no_such_kernel") is None
    assert bench.recorded_traffic("c2_glm_shared_indices", "no_such_schedule") is None
    assert bench.recorded_traffic("no_such_workload", "fused") is None


def test_launch_means_group_by_kernel():
    recs = [("resolve", 0.02), ("fused", 0.2), ("resolve", 0.03)]
    assert bench.launch_means_ms(recs) == {"resolve": [0.02, 0.03], "fused": [0.2]}


@pytest.mark.parametrize("n,g,sizes", [(8, 2, [4, 4]), (8, 3, [3, 3, 2]), (1, 2, [1]),
                                       (5, (2, 3), [2, 3])])
def test_layer_groups(n, g, sizes):
    groups = layer_groups(n, g)
    assert [len(x) for x in groups] == sizes
    assert np.array_equal(np.concatenate(groups), np.arange(n))


def test_layer_groups_reject_bad_sizes():
    with pytest.raises(ValueError):
        layer_groups(4, (2, 1))
    with pytest.raises(ValueError):
        layer_groups(4, (4, 0))


def test_cpu_model_is_a_string():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_cpu_baseline_on_a_request_sample():
    """The CPU baseline runs the oracle on the first n requests only, and
    says so."""
    from synth import tiny
    cfg = tiny(5)
    out = bench.cpu_baseline(cfg, 2, budget_s=2.0, min_s=0.05, n_reqs=2)
    assert out["kind"] == "oracle" and out["unit"] == "rows/s" and out["value"] > 0
    assert "requests 0..1 of 4" in out["sample"] and out["cores"] <= 2
    full = bench.cpu_baseline(cfg, 2, budget_s=2.0, min_s=0.05)
    assert f"all {cfg.n_req} requests" in full["sample"]


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus above 1 exits at once with a message
    (before any GPU work)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
