"""Seeded sweep of small layer shapes, HIP layer vs the fp64 oracle (needs an MI355X).

Each case draws H, I (multiples of 128), E, K, T, the routing kind and a shared
expert from a fixed seed, so the sweep covers combinations the hand-written
cases do not (odd panel counts, K close to E, experts on both sides of the
light/heavy split, tails of every tile size, shared experts of other widths) while staying reproducible.
Same bar as the parity tests: bit-exact dispatch, max|err| <= tol * max|ref|.
Every case runs with canary bands around the handle's workspace buffers and
its output, which must come back untouched.
"""
import os

import numpy as np
import pytest
import torch

from gpu_util import (GUARD, check_dispatch, check_out_guard, compare, guarded_out, oracle_out, problem, say,
                      to_host_problem)
from moe_expert_ffn_afd_amd import afd

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("AFD_SWEEP_CASES", "8"))  # more for a wider one-off sweep


def draw_case(dtype: str, i: int) -> dict:
    rng = np.random.default_rng(1000 * (1 + ["f32", "bf16", "fp8", "w8a8"].index(dtype)) + i)
    H = 128 * int(rng.integers(1, 5))
    I = 128 * int(rng.integers(1, 5))
    E = int(rng.integers(2, 40))
    K = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(1, 400))
    routing = str(rng.choice(["uniform", "zipf"]))
    shared = I if rng.random() < 0.3 else 0
    if shared and rng.random() < 0.5:  # a shared expert of another width
        shared = 128 * int(rng.integers(1, 6))
    return dict(dtype=dtype, T=T, H=H, I=I, E=E, K=K, routing=routing, shared_inter=shared)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "w8a8"])
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shapes(dtype, i):
    cfg = draw_case(dtype, i)
    say("case", dtype, i, cfg)
    p = problem(cfg, seed=100 + i)
    layer = afd.Layer(p)
    layer.set_canaries(GUARD)
    buf, out = guarded_out(layer, cfg["T"])
    layer.forward(p["hidden"], p["hidden_scales"], p["ids"], p["weights"], out=out)
    torch.cuda.synchronize()
    check_out_guard(buf, cfg["T"], cfg["H"])
    assert layer.check_canaries() == 0
    check_dispatch(layer, p)
    ref = oracle_out(to_host_problem(p))
    compare(out, ref, dtype, what="%s #%d %s" % (dtype, i, cfg))
    layer.close()
