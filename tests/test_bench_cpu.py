"""bench.py's CPU baseline (the oracle timed on the host, all threads and one thread) on the
smallest workload: the fields the JSON line carries."""

import bench
import workloads


def test_cpu_baseline_fields():
    wl = workloads.CONFIGS["0"]
    r = bench.cpu_baseline(workloads.generate(wl), wl, 0.2, wl.P)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert 1 <= r["cores"] <= 16 and r["host_cores"] >= 1
    one = r["one_thread"]
    assert one["unit"] == "tokens/s" and one["value"] > 0 and "1 thread" in one["sample"]
