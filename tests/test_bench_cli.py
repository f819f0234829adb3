"""bench.py's host-side contract (no GPU): the one-GPU refusal and the traffic table's keys."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_traffic_entries_name_existing_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.TRAFFIC, "no recorded traffic figures"
    for key, t in bench.TRAFFIC.items():
        assert "/" in key, key
        path = os.path.join(ROOT, "context_attention_lse_amd", "csrc", t["source"])
        assert os.path.exists(path), (key, path)
        assert re.fullmatch(r"[0-9a-f]{16}", t["sha256"]), key
        assert t["fetch_kib"] > 0 and t["write_kib"] > 0, key
    # an unknown key reports no traffic rather than raising
    assert bench.traffic("no_such_kernel/no_such_workload") is None
