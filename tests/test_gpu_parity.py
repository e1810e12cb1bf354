"""HIP layer vs the fp64 oracle, through the C ABI (needs an MI355X).

Dispatch (counts, offsets, permutation, row map) must match bit for bit;
outputs within max|err| <= tol * max|ref| (bf16 2e-2, block-FP8 6e-2, fp32
1e-5).  Small cases run the whole batch through the oracle.  At full size the
tiny and decode workloads compare every token; the others compare the tokens
that hold the first and the last row of every m-tile of both tile lists (the
oracle computes tokens independently), plus the full dispatch.
"""
import numpy as np
import pytest
import torch

from gpu_util import (TOL, check_dispatch, compare, oracle_out, problem, run_layer, say, tile_covering_tokens,
                      to_host_problem)
from moe_expert_ffn_afd_amd import afd, inputs

pytestmark = pytest.mark.gpu


def small(dtype, T, H, I, E, K, routing="uniform", shared=0, global_experts=None):
    return dict(dtype=dtype, T=T, H=H, I=I, E=E, K=K, routing=routing, shared_inter=shared,
                global_experts=global_experts)


SMALL_CASES = {
    # name: (cfg, seed)
    "f32_tiny_full": (inputs.workload("tiny"), 0),
    "f32_ragged_shared": (small("f32", 45, 256, 384, 5, 3, shared=384), 1),
    "bf16_mr1_ragged": (small("bf16", 37, 256, 384, 16, 2), 2),
    "bf16_mr2_multi_tile": (small("bf16", 150, 512, 384, 6, 3), 3),
    "bf16_zipf_empty_experts": (small("bf16", 300, 256, 256, 16, 4, routing="zipf"), 4),
    "fp8_mr1": (small("fp8", 33, 512, 256, 16, 2), 5),
    "fp8_shared_multi_tile": (small("fp8", 70, 512, 384, 5, 3, shared=384), 6),
    "fp8_local_shard": (small("fp8", 200, 256, 384, 4, 8, routing="local_shard", global_experts=32), 7),
    # top-k at its limit (32) plus a shared expert: 33 rows per token in the combine; H = 384
    # leaves the last group of 8 down panels half full
    "bf16_k32_shared_h384": (small("bf16", 40, 384, 256, 64, 32, shared=256), 8),
    "fp8_k32_shared_h384": (small("fp8", 40, 384, 256, 64, 32, shared=256), 9),
    # heavy experts over several m-tiles with ragged last tiles (bf16: 256-row tiles,
    # block-FP8: 128-row tiles)
    "bf16_heavy_ragged": (small("bf16", 600, 256, 256, 4, 2), 10),
    "fp8_heavy_ragged": (small("fp8", 300, 256, 256, 4, 2), 11),
    # W8A8 (int8 MFMA, per-token and per-channel scales, h re-quantised per row)
    "w8a8_mr1": (small("w8a8", 33, 512, 256, 16, 2), 12),
    "w8a8_shared_multi_tile": (small("w8a8", 70, 512, 384, 5, 3, shared=384), 13),
    "w8a8_heavy_ragged": (small("w8a8", 300, 256, 256, 4, 2), 14),
    "w8a8_k32_shared_h384": (small("w8a8", 40, 384, 256, 64, 32, shared=256), 15),
    "w8a8_local_shard": (small("w8a8", 200, 256, 384, 4, 8, routing="local_shard", global_experts=32), 16),
    # a shared expert of another width than the routed experts: ceil(Is / I)
    # parts of width I, the last zero-padded (twice, half, one and a half, three
    # times the routed width; light and heavy shared tiles)
    "bf16_shared_2x": (small("bf16", 60, 256, 256, 8, 2, shared=512), 17),
    "bf16_shared_2x_heavy": (small("bf16", 600, 256, 256, 4, 2, shared=512), 18),
    "fp8_shared_half": (small("fp8", 70, 512, 256, 5, 3, shared=128), 19),
    "fp8_shared_1p5x_heavy": (small("fp8", 300, 256, 256, 6, 2, shared=384), 20),
    "w8a8_shared_3x": (small("w8a8", 50, 256, 128, 6, 2, shared=384), 21),
    "f32_shared_1p5x": (small("f32", 45, 256, 256, 5, 3, shared=384), 22),
    # block-FP8 and W8A8 batches of at least 128 routed rows per expert on
    # average: the experts of more than 128 rows (and the shared expert) take
    # the LDS-tiled 8-bit GEMM's 256-row tiles, ragged last tiles included;
    # with Zipf routing all three lists (tiled, 128-row heavy, 64-row light)
    # in one stage; 150 rows per expert on average put experts on both sides
    # of 128 rows
    "fp8_tiled_ragged": (small("fp8", 700, 256, 384, 4, 2), 23),
    "fp8_tiled_shared_parts": (small("fp8", 600, 512, 256, 4, 2, shared=384), 24),
    "fp8_tiled_three_lists": (small("fp8", 1100, 256, 256, 16, 4, routing="zipf"), 25),
    "w8a8_tiled_ragged": (small("w8a8", 700, 256, 384, 4, 2), 26),
    "w8a8_tiled_three_lists": (small("w8a8", 1100, 256, 256, 16, 4, routing="zipf"), 27),
    "fp8_tiled_about_128_rows": (small("fp8", 600, 256, 384, 8, 2, shared=256), 28),
    "w8a8_tiled_about_128_rows": (small("w8a8", 600, 256, 384, 8, 2), 29),
}


@pytest.mark.parametrize("name", sorted(SMALL_CASES))
def test_small_full_batch(name):
    cfg, seed = SMALL_CASES[name]
    say("case", name, cfg, "seed", seed)
    p = problem(cfg, seed)
    layer, out = run_layer(p)
    check_dispatch(layer, p)
    ref = oracle_out(to_host_problem(p))
    compare(out, ref, cfg["dtype"], what=name)
    layer.close()


FULL = ["tiny", "decode", "aggregated", "fp8_shared", "w8a8_shared"]
EVERY_TOKEN = {"tiny", "decode"}


def covering(cfg, ids, max_tiles=None):
    """Tokens covering the first and last row of every m-tile (see gpu_util)."""
    tokens, cov = tile_covering_tokens(cfg["dtype"], ids.shape[0], cfg["E"], cfg["K"], ids,
                                       bool(cfg.get("shared_inter")), max_tiles=max_tiles)
    say("  compared tiles (compared, of): %s; %d tokens" % (cov, len(tokens)))
    return tokens


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    cfg = inputs.workload(name)
    say("workload", name, inputs.WORKLOAD_TITLES[name])
    p = problem(cfg, 0)
    layer, out = run_layer(p)
    check_dispatch(layer, p)
    ids = p["ids"].cpu().numpy()
    tokens = None if name in EVERY_TOKEN else covering(cfg, ids)
    ref = oracle_out(to_host_problem(p), tokens)
    compare(out, ref, cfg["dtype"], tokens=tokens, what=name)
    # rows with no local expert and no shared expert are exactly zero
    empty = np.where((ids < 0).all(axis=1))[0]
    if len(empty) and not cfg.get("shared_inter"):
        assert torch.all(out[torch.from_numpy(empty).cuda()] == 0)
    layer.close()


LARGEST = {
    # the largest batches of the batch-size sweep: 131072 routed rows; with the
    # shared expert the down outputs (147456 rows of 7168 bf16) sit just under
    # the 2 GiB of 32-bit buffer offsets
    "bf16_uniform_T16384": inputs.workload("decode", T=16384),
    "bf16_zipf_T16384": inputs.workload("aggregated", T=16384),
    "fp8_shared_T16384": inputs.workload("fp8_shared", T=16384),
    "w8a8_shared_T16384": inputs.workload("w8a8_shared", T=16384),
    # 128 routed rows per expert on average: every expert of more than one
    # 128-row ring tile takes a 256-row tiled tile
    "fp8_shared_T4096": inputs.workload("fp8_shared", T=4096),
}
# tiles per list whose first and last rows are compared (None: all); the
# 8-bit oracle takes about 7 core-seconds per token of that shape
LARGEST_TILES = {"bf16_uniform_T16384": None, "bf16_zipf_T16384": None, "fp8_shared_T16384": 40,
                 "w8a8_shared_T16384": 16, "fp8_shared_T4096": 24}


@pytest.mark.parametrize("name", sorted(LARGEST))
def test_largest_batches(name):
    cfg = LARGEST[name]
    say("largest batch", name, cfg)
    p = problem(cfg, 0)
    layer, out = run_layer(p)
    check_dispatch(layer, p)
    T = cfg["T"]
    tokens = np.union1d(covering(cfg, p["ids"].cpu().numpy(), LARGEST_TILES[name]), [0, 1, T - 2, T - 1])
    ref = oracle_out(to_host_problem(p), tokens)
    compare(out, ref, cfg["dtype"], tokens=tokens, what=name)
    layer.close()


PING_PONG = {
    # the speculative-verify shard at full size (block-FP8 ring GEMMs)
    "verify_shard": inputs.workload("verify_shard"),
    # bf16 with Zipf routing: each microbatch has heavy and light experts, so
    # both run the mixed launch (on all CUs, then on half of them)
    "bf16_zipf_mixed": small("bf16", 2048, 1024, 512, 32, 8, routing="zipf"),
}


@pytest.mark.parametrize("name", sorted(PING_PONG))
def test_two_streams_ping_pong(name):
    """Two microbatches on two streams (clone shares weights) equal the
    one-call result bit for bit, and match the oracle on sampled tokens."""
    cfg = PING_PONG[name]
    say("ping-pong", name, cfg)
    p = problem(cfg, 0)
    T = cfg["T"]
    half = T // 2
    l0 = afd.Layer(p, max_tokens=T)
    l1 = l0.clone()
    single = l0.forward(p["hidden"], p["hidden_scales"], p["ids"], p["weights"])
    torch.cuda.synchronize()
    check_dispatch(l0, p)  # the single call over all T tokens
    mbs = [inputs.slice_tokens(p, 0, half), inputs.slice_tokens(p, half, T)]
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    runs = []
    for conc in (1, 2):  # whole-device grids, then each call on half the CUs
        say("concurrency", conc)
        l0.set_concurrency(conc)
        l1.set_concurrency(conc)
        outs = [l0.out_like(half), l1.out_like(half)]
        torch.cuda.synchronize()
        for layer, mb, st, o in ((l0, mbs[0], s0, outs[0]), (l1, mbs[1], s1, outs[1])):
            with torch.cuda.stream(st):
                layer.forward(mb["hidden"], mb["hidden_scales"], mb["ids"], mb["weights"], out=o, stream=st)
        torch.cuda.synchronize()
        runs.append(torch.cat(outs))
    assert torch.equal(runs[0], runs[1]), "the CU share changed the result"
    pp = runs[1]
    assert torch.equal(pp, single), "ping-pong microbatches differ from the single call"
    check_dispatch(l0, mbs[0])
    check_dispatch(l1, mbs[1])
    local = (p["ids"] >= 0).float().mean().item()
    say("  local hit fraction %.3f" % local)
    # every m-tile of the single call and of both microbatches (whose outputs
    # equal the single call's bit for bit)
    ids = p["ids"].cpu().numpy()
    say("  single call:")
    tokens = covering(cfg, ids)
    for i, mb in enumerate(mbs):
        say("  microbatch %d:" % i)
        tokens = np.union1d(tokens, covering(cfg, mb["ids"].cpu().numpy()) + i * half)
    ref = oracle_out(to_host_problem(p), tokens)
    compare(single, ref, cfg["dtype"], tokens=tokens, what=name)
    l1.close()
    l0.close()
