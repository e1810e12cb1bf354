"""The layer's forward captured in a HIP graph: the forward makes no allocation,
no synchronisation and no memset, so one capture replays the whole layer
(dispatch, both grouped GEMMs, combine).  Every replay, with eager forwards of
another batch on the same handle in between (they overwrite its workspace),
must give the eager result bit for bit, and that result matches the oracle."""
import pytest
import torch

from gpu_util import compare, oracle_out, problem, say, to_host_problem
from moe_expert_ffn_afd_amd import afd, inputs

pytestmark = pytest.mark.gpu


def cfg(dtype, T, H, I, E, K, routing="uniform", shared=0):
    return dict(dtype=dtype, T=T, H=H, I=I, E=E, K=K, routing=routing, shared_inter=shared, global_experts=None)


CASES = {
    "bf16_light_only": (cfg("bf16", 64, 512, 256, 16, 2), 21),
    "bf16_zipf_mixed": (cfg("bf16", 700, 512, 256, 8, 4, routing="zipf"), 22),
    "fp8_shared_ring": (cfg("fp8", 150, 512, 384, 6, 3, shared=384), 23),
    "w8a8_shared_ring": (cfg("w8a8", 150, 512, 384, 6, 3, shared=384), 25),
    "f32_tiny": (cfg("f32", 40, 256, 384, 5, 3), 24),
}


def fwd(layer, q, out):
    layer.forward(q["hidden"], q["hidden_scales"], q["ids"], q["weights"], out=out,
                  stream=torch.cuda.current_stream())


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_eager(name):
    c, seed = CASES[name]
    say("graph case", name, c, "seed", seed)
    p = problem(c, seed)
    other = problem(c, seed + 100)
    layer = afd.Layer(p)
    eager = layer.out_like(c["T"])
    fwd(layer, p, eager)
    torch.cuda.synchronize()
    compare(eager, oracle_out(to_host_problem(p)), c["dtype"], what=name)

    out = layer.out_like(c["T"])
    scratch = layer.out_like(c["T"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(layer, p, out)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd(layer, p, out)
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        fwd(layer, other, scratch)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say("replay", r)
        assert torch.equal(out, eager), "replay %d differs from the eager forward" % r
    del graph
    layer.close()


def test_graph_of_two_stream_ping_pong():
    """Two microbatches on two streams (a handle and its clone), forked from
    and joined to the capture stream inside one graph: every replay equals
    the eager two-stream result bit for bit."""
    c = cfg("fp8", 256, 512, 256, 8, 4, routing="uniform")
    p = problem(c, 31)
    half = c["T"] // 2
    parts = [inputs.slice_tokens(p, i * half, (i + 1) * half) for i in range(2)]
    layers = [afd.Layer(p, max_tokens=half)]
    layers.append(layers[0].clone())
    for layer in layers:
        layer.set_concurrency(2)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]

    def step(outs):
        main = torch.cuda.current_stream()
        for i in range(2):
            streams[i].wait_stream(main)
            with torch.cuda.stream(streams[i]):
                fwd(layers[i], parts[i], outs[i])
        for i in range(2):
            main.wait_stream(streams[i])

    eager = [layers[i].out_like(half) for i in range(2)]
    step(eager)
    torch.cuda.synchronize()
    ref = oracle_out(to_host_problem(p))
    compare(torch.cat(eager), ref, "fp8", what="two-stream eager")

    outs = [layers[i].out_like(half) for i in range(2)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(outs)
    torch.cuda.synchronize()
    for r in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say("two-stream replay", r)
        for i in range(2):
            assert torch.equal(outs[i], eager[i]), "replay %d, microbatch %d differs" % (r, i)
    del graph
    for layer in layers[::-1]:
        layer.close()
