"""bench.py host-side contract: one GPU only, and the traffic bookkeeping."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_scales_and_entries():
    # FETCH_SIZE reads half of a plain copy's bytes, WRITE_SIZE all of them
    assert abs(bench.FETCH_SCALE - 2.0) < 1e-3 and bench.WRITE_SCALE == 1.0
    for name, t in bench.TRAFFIC.items():
        assert set(t) == {"sources", "sha", "fetch_kib", "write_kib"}, name
        assert len(t["sha"]) == 16 and t["fetch_kib"] > 0 and t["write_kib"] > 0
        for src in t["sources"]:
            assert os.path.exists(os.path.join(ROOT, "expert_routed_ffn_amd", "csrc", src)), src
        got = bench.measured_traffic(name)
        # null once the kernel sources differ from the ones the counters were taken on
        if bench._sources_sha(t["sources"]) == t["sha"]:
            assert got == (t["fetch_kib"] * bench.FETCH_SCALE + t["write_kib"]) * 1024.0
        else:
            assert got is None
    assert bench.measured_traffic("no_such_kernel") is None
