"""afd_ffn_forward_noalloc, the forward whose workspace is the library's static
device scratch, against afd_ffn_forward on the same handle: the same kernels on
the same inputs, so outputs must agree bit for bit.  Two calls in a row, the
second with fewer tokens (the scratch keeps the first call's contents), then a
size past the scratch, which must be refused on the host."""
import numpy as np
import pytest
import torch

from gpu_util import compare, oracle_out, problem, say, to_host_problem
from moe_expert_ffn_afd_amd import afd, inputs

pytestmark = pytest.mark.gpu


def cfg(dtype, T, H, I, E, K, routing="uniform", shared=0):
    return dict(dtype=dtype, T=T, H=H, I=I, E=E, K=K, routing=routing, shared_inter=shared, global_experts=None)


CASES = {
    # (config of the first call, tokens of the second call, seed)
    "bf16_mixed": (cfg("bf16", 300, 1024, 512, 32, 8, routing="zipf"), 70, 31),
    "bf16_light_only": (cfg("bf16", 64, 512, 256, 16, 4), 9, 32),
    "fp8_shared": (cfg("fp8", 160, 512, 384, 8, 4, shared=384), 33, 33),
    "f32_tiny": (inputs.workload("tiny"), 20, 34),
}


def both(layer, q):
    ref = layer.out_like(q["T"])
    got = layer.out_like(q["T"])
    got.fill_(float("nan"))
    st = torch.cuda.current_stream()
    afd.afd_ffn_forward(layer.handle, q["T"], q["hidden"], q["hidden_scales"], q["ids"], q["weights"], ref, st)
    afd.afd_ffn_forward_noalloc(layer.handle, q["T"], q["hidden"], q["hidden_scales"], q["ids"], q["weights"],
                                got, st)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("name", sorted(CASES))
def test_noalloc_matches_forward(name):
    c, t2, seed = CASES[name]
    say("no-alloc case", name, c, "second T", t2, "seed", seed)
    p = problem(c, seed)
    layer = afd.Layer(p)
    ref, got = both(layer, p)
    assert torch.equal(ref, got), "first call: the no-alloc forward differs from afd_ffn_forward"
    # second call, smaller, on other tokens of another batch: the scratch still
    # holds the first call's dispatch, h and y
    other = problem(c, seed + 1000)
    mixed = dict(p, hidden=other["hidden"], hidden_scales=other["hidden_scales"], ids=other["ids"],
                 weights=other["weights"])
    q = inputs.slice_tokens(mixed, 5, 5 + t2)
    ref2, got2 = both(layer, q)
    assert torch.equal(ref2, got2), "second call: the no-alloc forward differs from afd_ffn_forward"
    compare(got2, oracle_out(to_host_problem(q)), c["dtype"], what=name + " second call vs oracle")
    layer.close()


def test_noalloc_refuses_more_than_the_scratch():
    # 8 rows of 512 + 1024 bf16 outputs per token: 3000 tokens need ~ 90 MiB
    c = cfg("bf16", 3000, 1024, 512, 16, 8)
    p = problem(c, 35)
    layer = afd.Layer(p)
    out = layer.out_like(c["T"])
    with pytest.raises(afd.AfdError) as e:
        afd.afd_ffn_forward_noalloc(layer.handle, c["T"], p["hidden"], None, p["ids"], p["weights"], out)
    assert e.value.status == afd.AFD_ERR_UNSUPPORTED
    say("  refused:", str(e.value))
    # a size that fits still runs after the refusal
    q = inputs.slice_tokens(p, 0, 100)
    ref, got = both(layer, q)
    assert torch.equal(ref, got)
    assert np.isfinite(got.float().cpu().numpy()).all()
    layer.close()
