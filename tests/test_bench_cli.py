"""CPU tests of bench.py's command line: it refuses more than one GPU with a
message, and its host-only planner workload (join-order search latency) runs
and prints one JSON line without a GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_search_workload_runs_on_the_host():
    r = _run("--workload", "search")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    out = json.loads(lines[0])
    assert out["unit"] == "ms"
    assert set(out["queries"]) == {"4", "8", "10", "12"}
    for q in out["queries"].values():
        assert q["median_ms"] >= 0 and len(q["frontier_sizes"]) == 5
        assert all(f >= 1 for f in q["frontier_sizes"])


def test_executed_projection_flops_count_the_pruned_last_layer():
    """The FLOP figures count what runs: every layer but the last for every
    token, the last layer's QKV for every token, its O projection and MLP for
    the pairs' last rows only. The per-layer figures are the Qwen3-4B matrix
    shapes."""
    sys.path.insert(0, ROOT)
    import bench
    qkv = 2 * 2560 * (32 + 2 * 8) * 128
    layer = qkv + 2 * 4096 * 2560 + 2 * 2560 * 2 * 9728 + 2 * 9728 * 2560
    assert bench.GEMM_FLOP_QKV == qkv and bench.GEMM_FLOP_LAYER == layer
    # one layer, every suffix token a pair's last row: the whole layer each
    assert bench.executed_gemm_flops(1, 10, 10, 0) == 10 * layer
    # 36 layers, 64-token suffixes: 64 tokens x 35 layers + 64 QKV + 1 tail
    got = bench.executed_gemm_flops(36, 64 * 3, 3, 5)
    want = (64 * 3 + 5) * (35 * layer + qkv) + 3 * (layer - qkv)
    assert got == want
