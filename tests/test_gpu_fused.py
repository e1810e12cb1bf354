"""The whole layer in one persistent launch (afd_ffn_set_fused) on the GPU.

Every case runs the same batch through the separate launches and through the
fused launch on one handle: the outputs and the dispatch must be equal bit for
bit (the same per-element arithmetic), the dispatch must match the oracle bit
for bit and the outputs the oracle within the dtype's tolerance, and no grid
barrier may have timed out."""
import numpy as np
import pytest
import torch

from gpu_util import (check_dispatch, compare, oracle_out, problem, say, tile_covering_tokens,
                      to_host_problem)
from moe_expert_ffn_afd_amd import afd, inputs

pytestmark = pytest.mark.gpu


def cfg(dtype, T, H, I, E, K, routing="uniform", shared=0, global_experts=None):
    return dict(dtype=dtype, T=T, H=H, I=I, E=E, K=K, routing=routing, shared_inter=shared,
                global_experts=global_experts)


def run(layer, q, fused):
    layer.set_fused(fused)
    out = layer.forward(q["hidden"], q["hidden_scales"], q["ids"], q["weights"])
    torch.cuda.synchronize()
    return out, layer.dispatch(q["T"])


def fused_vs_separate(layer, q, what):
    ref, dref = run(layer, q, False)
    got, dgot = run(layer, q, True)
    for k in dref:
        assert np.array_equal(dref[k], dgot[k]), "%s: fused dispatch %s differs" % (what, k)
    assert torch.equal(ref, got), "%s: fused output differs from the separate launches" % what
    assert afd.afd_ffn_fused_errors(layer.handle) == 0, "%s: grid-barrier waits timed out" % what
    return got


CASES = {
    "fp8_light_only": (cfg("fp8", 33, 512, 256, 16, 2), 41),
    "fp8_shared_multi_tile": (cfg("fp8", 150, 512, 384, 6, 3, shared=384), 42),
    "fp8_heavy_ragged": (cfg("fp8", 300, 256, 256, 4, 2), 43),
    "fp8_local_shard": (cfg("fp8", 200, 256, 384, 4, 8, routing="local_shard", global_experts=32), 44),
    "fp8_k32_many_experts": (cfg("fp8", 40, 384, 256, 512, 32, shared=256), 45),
    "fp8_one_token": (cfg("fp8", 1, 256, 256, 8, 2, shared=256), 46),
    "w8a8_shared_multi_tile": (cfg("w8a8", 150, 512, 384, 6, 3, shared=384), 47),
    "w8a8_zipf": (cfg("w8a8", 700, 512, 256, 8, 4, routing="zipf"), 48),
    "fp8_shared_2p5x": (cfg("fp8", 150, 512, 256, 6, 3, shared=640), 53),
    # block-FP8 with the LDS-tiled list (experts of 256 rows or more) beside
    # the ring's heavy and light lists
    "fp8_tiled_three_lists": (cfg("fp8", 1100, 256, 256, 16, 4, routing="zipf", shared=256), 60),
    "w8a8_tiled_three_lists": (cfg("w8a8", 1100, 256, 256, 16, 4, routing="zipf", shared=256), 61),
    # bf16: the dispatch keeps every expert light (light-only streaming, 32-
    # and 64-row tiles), chooses the mixed split for a skewed batch, or always
    # takes it (shared expert, many rows per expert)
    "bf16_light_only_mr1": (cfg("bf16", 64, 512, 256, 32, 4), 54),
    "bf16_light_only_mr2": (cfg("bf16", 200, 256, 384, 32, 4), 55),
    "bf16_auto_zipf": (cfg("bf16", 256, 256, 256, 32, 4, routing="zipf"), 56),
    "bf16_heavy_ragged": (cfg("bf16", 600, 256, 256, 4, 2), 57),
    "bf16_shared_mixed": (cfg("bf16", 150, 512, 384, 6, 3, shared=384), 58),
    "bf16_shared_2x_heavy": (cfg("bf16", 600, 256, 256, 4, 2, shared=512), 59),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_equals_separate_launches(name):
    c, seed = CASES[name]
    say("fused case", name, c, "seed", seed)
    p = problem(c, seed)
    layer = afd.Layer(p)
    got = fused_vs_separate(layer, p, name)
    check_dispatch(layer, p)
    compare(got, oracle_out(to_host_problem(p)), c["dtype"], what=name + " fused")
    # repeated fused calls (the barrier state resets itself), another batch in between
    other = problem(c, seed + 500)
    q = dict(p, hidden=other["hidden"], hidden_scales=other["hidden_scales"], ids=other["ids"],
             weights=other["weights"])
    fused_vs_separate(layer, q, name + " second batch")
    again, _ = run(layer, p, True)
    assert torch.equal(again, got), "fused call not repeatable"
    layer.close()


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_fused_on_shares_of_the_cus(dtype):
    """Grids of a third of the CUs (not a multiple of the 8 XCDs) and of two."""
    c = cfg(dtype, 260, 512, 256, 16, 4, shared=256)
    p = problem(c, 49)
    layer = afd.Layer(p)
    base, _ = run(layer, p, False)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for share in (3, cus // 2):
        say("concurrency", share)
        layer.set_concurrency(share)
        got, _ = run(layer, p, True)
        assert torch.equal(got, base), "fused on 1/%d of the CUs differs" % share
        assert afd.afd_ffn_fused_errors(layer.handle) == 0
    layer.close()


def test_fused_refused_for_f32():
    p = problem(cfg("f32", 8, 256, 256, 4, 2), 50)
    layer = afd.Layer(p)
    with pytest.raises(afd.AfdError) as e:
        layer.set_fused(True)
    assert e.value.status == afd.AFD_ERR_UNSUPPORTED
    layer.close()


@pytest.mark.parametrize("name", ["fp8_shared", "w8a8_shared", "decode", "aggregated"])
def test_fused_full_size(name):
    c = inputs.workload(name)
    say("fused full size", name)
    p = problem(c, 0)
    layer = afd.Layer(p)
    got = fused_vs_separate(layer, p, name)
    check_dispatch(layer, p)
    # bit-equal to the separate launches, which the parity tests compare over
    # every m-tile; here a tile-covering sample of 40 tiles per list
    tokens, cov = tile_covering_tokens(c["dtype"], c["T"], c["E"], c["K"], p["ids"].cpu().numpy(),
                                       bool(c.get("shared_inter")), max_tiles=40)
    say("  compared tiles", cov, len(tokens), "tokens")
    compare(got, oracle_out(to_host_problem(p), tokens), c["dtype"], tokens=tokens, what=name + " fused")
    layer.close()


PING_PONG = {
    "verify_shard": inputs.workload("verify_shard"),
    # bf16 with Zipf routing: each microbatch has heavy and light experts
    "bf16_zipf_mixed": cfg("bf16", 2048, 1024, 512, 32, 8, routing="zipf"),
}


@pytest.mark.parametrize("name", sorted(PING_PONG))
def test_fused_two_stream_ping_pong(name):
    """Two microbatches, each one fused launch on half the CUs, running at once
    on two streams: equal to the single separate-launch call over all
    tokens."""
    c = PING_PONG[name]
    say("fused ping-pong", name)
    p = problem(c, 0)
    T = c["T"]
    half = T // 2
    l0 = afd.Layer(p, max_tokens=T)
    l1 = l0.clone()
    single, _ = run(l0, p, False)
    mbs = [inputs.slice_tokens(p, 0, half), inputs.slice_tokens(p, half, T)]
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    for layer in (l0, l1):
        layer.set_concurrency(2)
        layer.set_fused(True)
    outs = [l0.out_like(half), l1.out_like(half)]
    torch.cuda.synchronize()
    for layer, mb, st, o in ((l0, mbs[0], s0, outs[0]), (l1, mbs[1], s1, outs[1])):
        with torch.cuda.stream(st):
            layer.forward(mb["hidden"], mb["hidden_scales"], mb["ids"], mb["weights"], out=o, stream=st)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs), single), "fused ping-pong differs from the single call"
    assert afd.afd_ffn_fused_errors(l0.handle) == 0 and afd.afd_ffn_fused_errors(l1.handle) == 0
    check_dispatch(l0, mbs[0])
    check_dispatch(l1, mbs[1])
    tokens = np.sort(np.random.default_rng(8).choice(T, 16, replace=False))
    compare(single, oracle_out(to_host_problem(p), tokens), c["dtype"], tokens=tokens, what=name + " fused")
    l1.close()
    l0.close()


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_fused_graph_replay(dtype):
    """The fused forward captured in a HIP graph replays bit-exactly, with
    eager fused forwards of another batch on the same handle in between."""
    c = cfg(dtype, 150, 512, 384, 6, 3, shared=384)
    p = problem(c, 51)
    other = problem(c, 52)
    layer = afd.Layer(p)
    layer.set_fused(True)
    eager = layer.out_like(c["T"])
    layer.forward(p["hidden"], p["hidden_scales"], p["ids"], p["weights"], out=eager,
                  stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    replay_out = layer.out_like(c["T"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        layer.forward(p["hidden"], p["hidden_scales"], p["ids"], p["weights"], out=replay_out,
                      stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    scratch = layer.out_like(c["T"])
    for i in range(3):
        replay_out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(replay_out, eager), "replay %d differs" % i
        layer.forward(other["hidden"], other["hidden_scales"], other["ids"], other["weights"], out=scratch)
        torch.cuda.synchronize()
    assert afd.afd_ffn_fused_errors(layer.handle) == 0
    compare(eager, oracle_out(to_host_problem(p)), dtype, what="graph fused")
    del graph
    layer.close()
