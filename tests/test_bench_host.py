"""Host-side checks of bench.py: the one-GPU guard, the algorithmic units and the check of a measured run."""
import importlib.util
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_units_hand_counted():
    b = _bench()
    # 3 tokens, top-2 over 4 experts; expert 3 empty, one dropped slot (-1)
    ids = np.array([[0, 1], [1, -1], [2, 0]], dtype=np.int32)
    T, H, I, E, K = 3, 8, 16, 4, 2
    cfg = dict(T=T, H=H, I=I, E=E, K=K, dtype="bf16")
    u = b.algorithmic_units(cfg, ids)
    assert u["N"] == 5 and u["Ns"] == 5 and u["nonempty"] == 3
    assert u["gu_bytes"] == 3 * 2 * H * I * 2 + T * H * 2 + 5 * I * 2
    assert u["dn_bytes"] == 3 * I * H * 2 + 5 * I * 2 + 5 * H * 2
    assert u["layer_bytes"] == 3 * 3 * H * I * 2 + T * H * 2 + T * H * 2 + T * K * 8
    assert u["gu_flops"] == 4.0 * H * I * 5 and u["layer_flops"] == 6.0 * H * I * 5

    # a shared expert adds T rows and one always-read expert; FP8 adds scales
    cfg = dict(T=T, H=128, I=128, E=E, K=K, dtype="fp8", shared_inter=128)
    u = b.algorithmic_units(cfg, ids)
    assert u["Ns"] == 5 + T and u["nonempty"] == 4
    w = 128 * 128 * (1 + 4.0 / (128 * 128))
    assert abs(u["gu_bytes"] - (4 * 2 * w + T * 128 * (1 + 4.0 / 128) + 8 * 128 * (1 + 4.0 / 128))) < 1e-6


def test_roofline_kernel_labels_follow_the_tile_policy():
    """The label bench.py puts on the roofline's kernel names the launch the
    library makes for that batch: streaming kernel alone for decode-sized bf16
    batches, the mixed heavy + light launch otherwise, the ring for block-FP8."""
    b = _bench()
    from moe_expert_ffn_afd_amd import inputs
    decode = b.gate_up_kernels(inputs.workload("decode"), 256)
    assert "gemm_grouped_kernel<true, 1>" in decode and "gemm_mixed_kernel<true, 1>" in decode
    assert "gemm_mixed_kernel<true, 2>" in b.gate_up_kernels(inputs.workload("aggregated"), 4096)
    # 17-32 rows per expert on average: 64-row light tiles, or the mixed launch with 32-row ones
    wider = b.gate_up_kernels(inputs.workload("decode"), 512)
    assert "gemm_grouped_kernel<true, 2>" in wider and "gemm_mixed_kernel<true, 1>" in wider
    # with a shared expert the mixed launch always runs
    assert "gemm_mixed_kernel<true, 1>" in b.gate_up_kernels(dict(inputs.workload("decode"), shared_inter=1536), 512)
    assert "gemm_ring_kernel<true>" in b.gate_up_kernels(inputs.workload("fp8_shared"), 2048)
    assert "gemm_f32_kernel<true>" in b.gate_up_kernels(inputs.workload("tiny"), 64)


def test_check_of_the_measured_run():
    """bench.py's check of a run: outputs of the sampled tokens against the
    oracle's within the tolerance, and each microbatch's dispatch bit for bit
    (here a stand-in for the layer handle returns a dispatch on the host)."""
    import torch

    from oracle import oracle as orc

    b = _bench()
    ids = np.array([[0, 2], [1, -1], [2, 0], [3, 3]], dtype=np.int32)
    cfg = {"dtype": "bf16", "E": 4}

    class Handle:
        def __init__(self, d):
            self.d = d

        def dispatch(self, T):
            return self.d

    q = {"T": 4, "ids": torch.from_numpy(ids)}
    good = orc.dispatch(ids, 4)
    ref = np.array([[1.0, -2.0], [0.5, 4.0]])
    out = torch.tensor([[1.0, -2.0], [0.5, 4.0], [9.0, 9.0], [9.0, 9.0]])
    c = b.check_run(cfg, out, ref, [Handle(good)], [q])
    assert c["ok"] and c["dispatch_exact"] and c["tokens"] == 2 and c["max_err_over_max_ref"] == 0.0
    # an error of 3 % of max|ref| is past the bf16 tolerance (2 %)
    c = b.check_run(cfg, out + torch.tensor([[0.0, 0.12], [0.0, 0.0], [0, 0], [0, 0]]), ref, [Handle(good)], [q])
    assert not c["ok"] and abs(c["max_err_over_max_ref"] - 0.03) < 1e-9
    # one moved row of the permutation fails the dispatch check
    bad = dict(good, sorted_assign=good["sorted_assign"][::-1].copy())
    c = b.check_run(cfg, out, ref, [Handle(bad)], [q])
    assert not c["ok"] and not c["dispatch_exact"]
    # non-finite outputs fail
    c = b.check_run(cfg, torch.tensor([[float("nan"), 0.0], [0.5, 4.0]]), ref, [Handle(good)], [q])
    assert not c["ok"]
