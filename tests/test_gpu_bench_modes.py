"""bench.py's modes on the GPU, at the tiny fp32 workload: a line with the
oracle's CPU baseline and the check of its own run, the step
replayed from a HIP graph (graph_ms_per_step next to the eager line) and the
batch-size sweep (one JSON line per T, every T of the sweep that fits; the
sweep's own path, one handle for the largest T running prefixes of one batch,
checked against the oracle)."""
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from gpu_util import check_dispatch, compare, oracle_out, say, to_host_problem
from moe_expert_ffn_afd_amd import inputs

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


def test_sweep_path_matches_oracle():
    """The sweep's handle (sized for T=16384) and batch, at the smallest and the
    largest T: dispatch bit-exact and every token against the oracle."""
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    cfg, sizes, p, layer = bench.sweep_setup("tiny", 0)
    ids = p["ids"].cpu().numpy()
    for T in (sizes[0], sizes[-1]):
        say("sweep prefix T =", T)
        q = inputs.slice_tokens(p, 0, T)
        out = layer.out_like(T)
        layer.forward(q["hidden"], q["hidden_scales"], q["ids"], q["weights"], out=out)
        torch.cuda.synchronize()
        check_dispatch(layer, q)
        assert int((ids[:T] >= 0).sum()) == bench.algorithmic_units(dict(cfg, T=T), ids[:T])["N"]
        compare(out, oracle_out(to_host_problem(q)), cfg["dtype"], what="sweep T=%d" % T)
        assert np.isfinite(out.cpu().numpy()).all()
    layer.close()


def test_default_line_checks_its_run():
    """With the oracle's CPU baseline on, a bench line checks its own run."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "5",
                        "--warmup", "2"], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    say("  check", d["check"], "cpu baseline", d["cpu_baseline"])
    assert d["check"]["ok"] and d["check"]["dispatch_exact"] and d["check"]["tokens"] == 64
    assert 0.0 <= d["check"]["max_err_over_max_ref"] <= 1e-5
    assert d["cpu_baseline"]["kind"] == "oracle" and d["cpu_baseline"]["value"] > 0


def test_mfma_ceiling_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--mfma-ceiling"], capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])["mfma_ceiling"]
    for dt in ("bf16", "fp8", "w8a8"):
        say("  mfma ceiling", dt, d[dt])
        # a real, sustained rate: above a tenth of the spec peak, below the spec peak at 2.4 GHz
        assert 0.1 < d[dt]["frac_of_spec"] <= 1.02 and 0.5 < d[dt]["clock_ghz"] < 2.6
    for k in ("bf16_tile_loop_fragments_in_registers", "bf16_tile_loop_with_lds_reads"):
        say("  mfma ceiling", k, d[k])
        assert 0.1 < d[k]["frac_of_spec"] <= 1.02 and 0.5 < d[k]["clock_ghz"] < 2.6
    # the LDS reads cost MFMA time: never faster than the same loop without them
    assert d["bf16_tile_loop_with_lds_reads"]["tflops"] <= 1.03 * d["bf16_tile_loop_fragments_in_registers"]["tflops"]
