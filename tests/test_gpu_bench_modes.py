"""bench.py's other modes on the GPU, at the tiny fp32 workload: the step
replayed from a HIP graph (graph_ms_per_step next to the eager line) and the
batch-size sweep (one JSON line per T, every T of the sweep that fits)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--no-cpu-baseline",
                        *args], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    return [json.loads(line) for line in r.stdout.strip().splitlines()]


def test_graph_mode_line():
    (d,) = run_bench("--graph", "--steps", "5", "--warmup", "2")
    assert d["ms_per_step"] > 0 and d["graph_ms_per_step"] > 0
    assert d["roofline"]["launch_ms"] > 0


def test_sweep_lines():
    lines = run_bench("--sweep", "--steps", "2", "--warmup", "1")
    assert [d["T"] for d in lines] == [64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384]
    for d in lines:
        assert d["routed_rows"] == 2 * d["T"] and d["ms_per_step"] > 0
