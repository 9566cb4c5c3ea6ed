"""Host-side contract of bench.py and of the binding's timing events (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    """The path runs on one GPU's share of experts: --gpus N > 1 exits with a message
    (and without touching a GPU)."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_stored_counters_name_their_workload_and_source():
    """The stored HBM counters carry the workload, the hash of the GEMM sources they
    were taken with (bench.py reports them only while it matches) and the command."""
    sys.path.insert(0, ROOT)
    import bench
    with open(bench.COUNTERS) as f:
        table = json.load(f)["workloads"]
    assert {"decode_fp8", "prefill_fp8_zipf"} <= set(table)
    for name, c in table.items():
        assert c["workload"] == name
        assert len(c["kernel_source_sha"]) == 16 and len(bench.kernel_source_hash()) == 16
        assert c["traffic_bytes_per_launch"] > 0 and "rocprofv3 --pmc" in c["command"]
        assert "FETCH_SIZE" in c["command"] and "WRITE_SIZE" in c["command"]


def test_timing_events_must_exist_before_a_launch():
    """torch creates an event at its first record; the timed legs refuse an event that
    has no HIP handle yet instead of passing a null event on."""
    torch = pytest.importorskip("torch")
    import mixture_experts_ffn_topk_amd as mx
    e = torch.cuda.Event(enable_timing=True)
    with pytest.raises(ValueError, match="recorded once"):
        mx._event_handles((e, e))
