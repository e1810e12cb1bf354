"""Edge cases and invariants of the HIP layer on the GPU (through the C ABI)."""
import numpy as np
import pytest
import torch

from gpu_util import check_dispatch, compare, oracle_out, problem, run_layer, run_layer_guarded, say, to_host_problem
from moe_expert_ffn_afd_amd import afd

pytestmark = pytest.mark.gpu


def cfg(dtype="bf16", T=64, H=256, I=256, E=8, K=2, shared=0):
    return dict(dtype=dtype, T=T, H=H, I=I, E=E, K=K, routing="uniform", shared_inter=shared)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "w8a8"])
def test_adversarial_routing(dtype):
    """All tokens on one expert (many m-tiles), duplicate ids, -1 slots, nothing local."""
    T, E, K = 130, 6, 3
    rng = np.random.default_rng(1)
    cases = {
        "one_hot_expert": np.full((T, K), 4, np.int32),
        "duplicates_and_minus1": rng.choice(np.array([-1, 0, 0, 2, 5], np.int32), size=(T, K)).astype(np.int32),
        "nothing_local": np.full((T, K), -1, np.int32),
    }
    for name, ids in cases.items():
        say("case", dtype, name)
        w = rng.uniform(0.0, 1.0, size=(T, K)).astype(np.float32)
        p = problem(cfg(dtype, T=T, E=E, K=K), seed=3, routing=(ids, w))
        layer, out = run_layer(p)
        check_dispatch(layer, p)
        ref = oracle_out(to_host_problem(p))
        if name == "nothing_local":
            assert torch.all(out == 0)
        else:
            compare(out, ref, dtype, what=name)
        layer.close()


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "w8a8"])
def test_empty_and_tiny_batches(dtype):
    p = problem(cfg(dtype, T=40, shared=256 if dtype != "bf16" else 0), seed=2)
    layer = afd.Layer(p, max_tokens=40)
    for T in (0, 1, 2, 40):
        say("case", dtype, "T =", T)
        q = {k: v for k, v in p.items()}
        for k in ("hidden", "hidden_scales", "ids", "weights"):
            if q[k] is not None:
                q[k] = p[k][:T].contiguous()
        q["T"] = T
        out = layer.forward(q["hidden"], q["hidden_scales"], q["ids"], q["weights"])
        torch.cuda.synchronize()
        assert out.shape == (T, 256)
        if T:
            check_dispatch(layer, q)
            compare(out, oracle_out(to_host_problem(q)), dtype, what="T=%d" % T)
    layer.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "w8a8"])
def test_largest_expert_count_and_top_k(dtype):
    """E = 512 local experts and top-32 (the limits the library accepts), with a
    shared expert for the 16-bit and 8-bit formats: 40 tokens make 1280
    assignments spread thinly over the experts (most hold 1-5 rows, some none),
    and a skewed batch puts hundreds on a few."""
    for routing, T, seed in (("uniform", 40, 71), ("zipf", 96, 72)):
        c = dict(dtype=dtype, T=T, H=256, I=256, E=512, K=32, routing=routing,
                 shared_inter=0 if dtype == "f32" else 256)
        say("case", c)
        p = problem(c, seed=seed)
        layer, out = run_layer(p)
        check_dispatch(layer, p)
        compare(out, oracle_out(to_host_problem(p)), dtype, what="E=512 K=32 " + routing)
        layer.close()


LARGEST_WIDTHS = {
    # H and I at the 8-bit formats' limit (128 scale blocks, int32 sums of
    # 16384 int8 products) and bf16 at the same widths; one width at its
    # limit with the other at its smallest
    # (tokens: the oracle takes about 1.5 core-seconds per token and expert
    # at 16384 x 16384)
    "fp8_H16384_I16384": ("fp8", 16384, 16384, 12),
    "w8a8_H16384_I16384": ("w8a8", 16384, 16384, 12),
    "bf16_H16384_I16384": ("bf16", 16384, 16384, 12),
    "fp8_H128_I16384": ("fp8", 128, 16384, 33),
    "bf16_H16384_I128": ("bf16", 16384, 128, 33),
}


@pytest.mark.parametrize("name", sorted(LARGEST_WIDTHS))
def test_largest_hidden_and_intermediate_widths(name):
    """The widest reductions the library accepts: top-2 of 3 experts, every
    token against the oracle, inside canary bands."""
    dtype, H, I, T = LARGEST_WIDTHS[name]
    c = dict(dtype=dtype, T=T, H=H, I=I, E=3, K=2, routing="uniform", shared_inter=0)
    say("case", name, c)
    p = problem(c, seed=81)
    layer, out = run_layer_guarded(p)
    check_dispatch(layer, p)
    compare(out, oracle_out(to_host_problem(p)), dtype, what=name)
    layer.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "w8a8"])
def test_widest_shared_expert(dtype):
    """A shared expert of 16 times the routed width (the most parts the
    library takes): 16 parts of width I added to every token in order."""
    c = dict(dtype=dtype, T=70, H=256, I=128, E=4, K=2, routing="uniform", shared_inter=16 * 128)
    say("case", c)
    p = problem(c, seed=82)
    layer, out = run_layer_guarded(p)
    check_dispatch(layer, p)
    compare(out, oracle_out(to_host_problem(p)), dtype, what="shared expert of 16 parts")
    layer.close()


def test_dispatch_either_side_of_the_single_launch_limit():
    """Up to 4096 flat slots one dispatch launch also places the slots; above it a
    second launch does.  Both must give the oracle's bit-exact dispatch."""
    c = dict(dtype="bf16", T=513, H=128, I=128, E=200, K=8, routing="zipf", zipf_s=1.2, shared_inter=0)
    p = problem(c, seed=11)
    layer = afd.Layer(p, max_tokens=513)
    for T in (511, 512, 513):
        say("case T =", T, "slots =", T * 8)
        q = {k: v for k, v in p.items()}
        for k in ("hidden", "hidden_scales", "ids", "weights"):
            if q[k] is not None:
                q[k] = p[k][:T].contiguous()
        q["T"] = T
        out = layer.forward(q["hidden"], q["hidden_scales"], q["ids"], q["weights"])
        torch.cuda.synchronize()
        check_dispatch(layer, q)
        compare(out, oracle_out(to_host_problem(q)), "bf16", what="T=%d" % T)
    layer.close()


def test_concurrency_bounds_checked():
    p = problem(cfg("bf16"), seed=1)
    layer = afd.Layer(p)
    for bad in (0, -1, 1 << 20):
        with pytest.raises(afd.AfdError):
            layer.set_concurrency(bad)
    layer.set_concurrency(3)  # a share that does not divide the CU count
    out = layer.forward(p["hidden"], p["hidden_scales"], p["ids"], p["weights"])
    torch.cuda.synchronize()
    compare(out, oracle_out(to_host_problem(p)), "bf16", what="concurrency 3")
    layer.close()


def round_robin_ids(T, E, K):
    """Slot k of token t -> expert (K t + k) % E: every expert gets T K / E rows (+-1)."""
    return ((np.arange(T)[:, None] * K + np.arange(K)[None, :]) % E).astype(np.int32)


@pytest.mark.parametrize("case", ["heavy_only", "light_only", "both", "both_on_a_share_of_3",
                                  "both_on_two_workgroups", "both_on_one_workgroup"])
def test_mixed_launch_role_split(case):
    """bf16 batches past the decode bound (more than 16 rows per expert on
    average) run one launch per GEMM whose workgroups the dispatch splits
    between the heavy (LDS-tiled) and the light (streaming) tile lists: all
    heavy, all light, both, both on a CU share that is not a multiple of 8,
    and both on grids of two workgroups and of one (which runs both lists)."""
    rng = np.random.default_rng(11)
    if case == "heavy_only":      # 128 rows on each of 8 experts: heavy tiles only
        c, routing = cfg("bf16", T=512, E=8, K=2), round_robin_ids(512, 8, 2)
    elif case == "light_only":    # 18-19 rows on each of 64 experts: light tiles only
        c, routing = cfg("bf16", T=600, E=64, K=2), round_robin_ids(600, 64, 2)
    else:                         # Zipf: a few heavy experts, many light ones
        c, routing = dict(dtype="bf16", T=513, H=256, I=256, E=32, K=4, routing="zipf", zipf_s=1.2,
                          shared_inter=0), None
    if routing is not None:
        routing = (routing, rng.uniform(0.0, 1.0, size=routing.shape).astype(np.float32))
    say("case", case)
    p = problem(c, seed=12, routing=routing)
    layer = afd.Layer(p)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if case == "both_on_a_share_of_3":
        layer.set_concurrency(3)
    elif case == "both_on_two_workgroups":
        layer.set_concurrency(cus // 2)
    elif case == "both_on_one_workgroup":
        layer.set_concurrency(cus)
    out = layer.forward(p["hidden"], p["hidden_scales"], p["ids"], p["weights"])
    torch.cuda.synchronize()
    check_dispatch(layer, p)
    compare(out, oracle_out(to_host_problem(p)), "bf16", what=case)
    layer.close()


def skewed_ids(T, E, K, rows0):
    """Expert 0 in slot 0 of the first rows0 tokens, every other slot spread
    round-robin over experts 1..E-1: expert 0 gets exactly rows0 rows."""
    f = np.arange(T)[:, None] * K + np.arange(K)[None, :]
    ids = 1 + f % (E - 1)
    ids[:rows0, 0] = 0
    return ids.astype(np.int32)


@pytest.mark.parametrize("T, case", [
    (128, "uniform"), (128, "largest_64_rows"), (128, "largest_65_rows"), (128, "largest_128_rows"),
    (128, "largest_128_rows_one_workgroup"),
    (256, "uniform"), (256, "largest_128_rows"), (256, "largest_129_rows"), (256, "largest_200_rows_one_workgroup")])
def test_small_batch_launch_chosen_on_device(T, case):
    """bf16 batches of at most 32 rows per expert on average: the dispatch
    keeps every expert light (streaming GEMM alone, 32-row tiles up to 16
    rows per expert on average, else 64-row tiles) while the largest expert
    has at most two light tiles of rows, and takes the mixed launch (32-row
    light tiles) beyond; both gated kernels are launched and one returns at
    once.  Each side of the boundary in both regimes (T=128: 16 rows per
    expert on average, T=256: 32), and grids of one workgroup."""
    E, K = 32, 4
    rng = np.random.default_rng(13)
    if case == "uniform":
        c, routing = cfg("bf16", T=T, E=E, K=K), round_robin_ids(T, E, K)
    else:
        rows0 = int(case.split("_")[1])
        c, routing = cfg("bf16", T=T, E=E, K=K), skewed_ids(T, E, K, rows0)
    routing = (routing, rng.uniform(0.0, 1.0, size=routing.shape).astype(np.float32))
    say("case", case)
    p = problem(c, seed=14, routing=routing)
    layer = afd.Layer(p)
    if case.endswith("one_workgroup"):
        layer.set_concurrency(torch.cuda.get_device_properties(0).multi_processor_count)
    out = layer.forward(p["hidden"], p["hidden_scales"], p["ids"], p["weights"])
    torch.cuda.synchronize()
    want = check_dispatch(layer, p)
    if case != "uniform":
        assert want["counts"][0] == int(case.split("_")[1])
    compare(out, oracle_out(to_host_problem(p)), "bf16", what=case)
    layer.close()


def test_unused_experts_poisoned_with_nan():
    T, E, K = 50, 8, 2
    rng = np.random.default_rng(4)
    ids = rng.choice(np.array([1, 3, 6], np.int32), size=(T, K)).astype(np.int32)
    w = rng.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    p = problem(cfg("bf16", T=T, E=E, K=K), seed=5, routing=(ids, w))
    _, base = run_layer(p)
    for name in ("w_gate", "w_up", "w_down"):
        t = p[name].clone()
        for e in (0, 2, 4, 5, 7):
            t[e] = float("nan")
        p[name] = t
    layer, out = run_layer(p)
    assert torch.all(torch.isfinite(out.float()))
    assert torch.equal(out, base)
    layer.close()


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "w8a8"])
def test_deterministic_and_permutation_equivariant(dtype):
    p = problem(cfg(dtype, T=96, E=8, K=2, shared=256 if dtype == "fp8" else 0), seed=6)
    layer, a = run_layer(p)
    b = layer.forward(p["hidden"], p["hidden_scales"], p["ids"], p["weights"])
    torch.cuda.synchronize()
    assert torch.equal(a, b), "run twice differs"
    perm = torch.from_numpy(np.random.default_rng(0).permutation(96)).cuda()
    q = dict(p)
    for k in ("hidden", "hidden_scales", "ids", "weights"):
        if q[k] is not None:
            q[k] = p[k][perm].contiguous()
    c = layer.forward(q["hidden"], q["hidden_scales"], q["ids"], q["weights"])
    torch.cuda.synchronize()
    assert torch.equal(c, a[perm]), "token permutation is not equivariant"
    layer.close()


def test_identical_experts_equal_dense_ffn():
    T, E, K = 64, 6, 3
    p = problem(cfg("bf16", T=T, E=E, K=K), seed=7)
    for name in ("w_gate", "w_up", "w_down"):
        p[name] = p[name][:1].expand_as(p[name]).contiguous()
    layer, out = run_layer(p)
    x = p["hidden"].double().cpu()
    wg, wu, wd = (p[n][0].double().cpu() for n in ("w_gate", "w_up", "w_down"))
    dense = ((torch.nn.functional.silu(x @ wg) * (x @ wu)) @ wd) * p["weights"].double().cpu().sum(1, keepdim=True)
    compare(out, dense.numpy(), "bf16", what="identical experts")
    layer.close()


def test_out_of_range_ids_are_counted_and_ignored():
    T, E, K = 20, 4, 2
    ids = np.zeros((T, K), np.int32)
    ids[3, 1] = 9
    ids[5, 0] = -5
    w = np.ones((T, K), np.float32) * 0.5
    p = problem(cfg("bf16", T=T, E=E, K=K), seed=8, routing=(ids, w))
    layer, out = run_layer(p)
    assert afd.afd_ffn_routing_errors(layer.handle) == 2
    ids2 = ids.copy()
    ids2[3, 1] = -1
    ids2[5, 0] = -1
    q = dict(p)
    q["ids"] = torch.from_numpy(ids2).cuda()
    _, ref = run_layer(q)
    assert torch.equal(out, ref)
    layer.close()


def test_forward_rejects_bad_shapes_on_host():
    p = problem(cfg("bf16", T=16), seed=9)
    layer = afd.Layer(p, max_tokens=16)
    with pytest.raises(ValueError):
        layer.forward(p["hidden"][:, :128].contiguous(), None, p["ids"], p["weights"])
    with pytest.raises(ValueError):
        layer.forward(p["hidden"], None, p["ids"].long(), p["weights"])
    big = torch.zeros((17, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        layer.forward(big, None, torch.zeros((17, 2), dtype=torch.int32, device="cuda"),
                      torch.zeros((17, 2), device="cuda"))
    lib = afd.load()
    st = lib.afd_ffn_forward(layer.handle, 17, None, None, None, None, None, None)
    assert st == afd.AFD_ERR_INVALID_ARG
    # misaligned device pointers are refused before anything is enqueued
    out = layer.out_like(16)
    h, ids, w = p["hidden"].data_ptr(), p["ids"].data_ptr(), p["weights"].data_ptr()
    for args in [(h + 2, ids, w, out.data_ptr()), (h, ids, w, out.data_ptr() + 8),
                 (h, ids + 2, w, out.data_ptr()), (h, ids, w + 1, out.data_ptr())]:
        st = lib.afd_ffn_forward(layer.handle, 16, args[0], None, args[1], args[2], args[3], None)
        assert st == afd.AFD_ERR_INVALID_ARG
        assert b"aligned" in lib.afd_ffn_last_error()
    torch.cuda.synchronize()
    layer.close()


def test_timing_records_every_stage():
    p = problem(cfg("bf16", T=64), seed=10)
    layer = afd.Layer(p)
    afd.afd_ffn_set_timing(layer.handle, True)
    for _ in range(3):
        layer.forward(p["hidden"], None, p["ids"], p["weights"])
    ms, n = afd.afd_ffn_get_timing(layer.handle)
    assert n == 3 and all(t > 0 for t in ms), ms
    # one stage only: the others read 0; a bit past the last stage is rejected
    afd.afd_ffn_set_timing_stages(layer.handle, [2])
    for _ in range(2):
        layer.forward(p["hidden"], None, p["ids"], p["weights"])
    ms, n = afd.afd_ffn_get_timing(layer.handle)
    assert n == 2 and ms[2] > 0 and all(ms[i] == 0 for i in (0, 1, 3, 4)), ms
    with pytest.raises(afd.AfdError):
        afd.afd_ffn_set_timing_stages(layer.handle, [afd.AFD_NUM_STAGES])
    afd.afd_ffn_set_timing(layer.handle, False)
    layer.forward(p["hidden"], None, p["ids"], p["weights"])
    ms, n = afd.afd_ffn_get_timing(layer.handle)
    assert n == 0 and all(t == 0 for t in ms), ms
    layer.close()
