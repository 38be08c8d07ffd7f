"""bench.py's contract, checked on the host: it runs on one GPU only, and the
stored HBM-traffic counters apply only to the kernel sources they were taken
on (the JSON line reports null for them otherwise)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (no GPU work at import)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus_requested"] == 2


def test_stored_traffic_matches_the_committed_kernels():
    with open(bench.TRAFFIC_FILE) as f:
        stored = json.load(f)
    for workload in ("gdn", "decode"):
        assert stored[workload]["gemm_source_sha"] == bench.gemm_source_sha(workload), \
            f"{workload}: kernel sources changed since the counters were taken; measure them again"
        assert bench.load_traffic(workload) == stored[workload]["hbm_bytes_per_launch"]


def test_traffic_is_null_once_the_kernel_changes(monkeypatch):
    monkeypatch.setattr(bench, "gemm_source_sha", lambda workload: "0" * 16)
    assert bench.load_traffic("gdn") is None
    assert bench.load_traffic("decode") is None


def test_stored_traffic_follows_from_its_counters():
    """hbm bytes = FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by
    what the counter read for a copy of known size; never below the
    algorithmic bytes of the launch."""
    with open(bench.TRAFFIC_FILE) as f:
        stored = json.load(f)
    for workload in ("gdn", "decode"):
        e = stored[workload]
        fetch = e["fetch_kib_per_dispatch"] * e["copy_bytes"] / e["copy_fetch_kib"]
        write = e["write_kib_per_dispatch"] * e["copy_bytes"] / e["copy_write_kib"]
        assert abs(fetch + write - e["hbm_bytes_per_launch"]) <= 1e-4 * e["hbm_bytes_per_launch"]
        assert e["hbm_bytes_per_launch"] >= 0.99 * e["algorithmic_bytes_per_launch"]
