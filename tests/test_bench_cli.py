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
