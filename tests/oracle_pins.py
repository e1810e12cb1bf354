"""Pins of the fp64 oracle against things other than itself.

Each pin takes a loaded oracle library (``oracle.oracle.load()`` or a
deliberately broken build of it) and raises AssertionError when the oracle
disagrees with:

* library routines: numpy's bincount / cumsum / stable argsort for the
  dispatch, torch's bf16, E4M3FN and int8 decoders, torch fp64 matrix
  products for the one-expert case (a plain SwiGLU FFN);
* a dense brute-force formulation on tiny inputs: every expert applied to
  every token, masked by a [T,E] routing-weight matrix (no gather, no per-slot
  loop, no shared code with the oracle);
* invariants of the layer: identical experts with weights summing to one give
  the dense FFN; token permutation permutes outputs; unused experts (poisoned
  with NaN) contribute nothing; linearity in the routing weights; zero input
  gives exactly zero;
* a closed form worked by hand (tests/golden/closed_form_swiglu.json).

``ALL_PINS`` lists them; tests/test_oracle.py runs them on the real oracle and
tests/test_oracle_mutants.py checks that each planted mistake trips one.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

from moe_expert_ffn_afd_amd import inputs
from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---- independent decoders (torch) and dense reference (numpy) -------------

def torch_decode(a, dtype):
    """fp64 numpy values of raw inputs via torch's own casts."""
    t = a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))
    t = t.cpu()
    if dtype == "f32":
        return t.double().numpy()
    if dtype == "bf16":
        return t.view(torch.bfloat16).double().numpy() if t.dtype != torch.bfloat16 else t.double().numpy()
    if dtype == "w8a8":
        return t.view(torch.int8).double().numpy()
    return t.view(torch.float8_e4m3fn).double().numpy()


def dequant(codes, scales, dtype):
    v = torch_decode(codes, dtype)
    if dtype not in ("fp8", "w8a8"):
        return v
    s = scales.cpu().double().numpy() if isinstance(scales, torch.Tensor) else np.asarray(scales, np.float64)
    if dtype == "w8a8":
        # one scale per output column, the same for every row of the matrix
        return v * np.expand_dims(s, -2)
    # expand the block grid over the last two axes
    s = np.repeat(np.repeat(s, 128, axis=-2), 128, axis=-1) if s.ndim >= 2 else s
    return v * s


def dense_reference(p):
    """y [T,H] fp64 = sum_e R[:,e] * FFN_e(X) (+ shared), all experts on all tokens."""
    dt = p["dtype"]
    X = torch_decode(p["hidden"], dt)
    if dt == "fp8":
        hs = p["hidden_scales"].cpu().double().numpy()
        X = X * np.repeat(hs, 128, axis=1)
    if dt == "w8a8":
        X = X * p["hidden_scales"].cpu().double().numpy()[:, None]
    Wg = dequant(p["w_gate"], p["s_gate"], dt)
    Wu = dequant(p["w_up"], p["s_up"], dt)
    Wd = dequant(p["w_down"], p["s_down"], dt)
    ids = p["ids"].cpu().numpy()
    w = p["weights"].cpu().double().numpy()
    T, K = ids.shape
    E = Wg.shape[0]
    R = np.zeros((T, E))
    for e in range(E):
        R[:, e] = np.where(ids == e, w, 0.0).sum(axis=1)
    G = np.einsum("th,ehi->eti", X, Wg)
    U = np.einsum("th,ehi->eti", X, Wu)
    A = G / (1.0 + np.exp(-G)) * U
    F = np.einsum("eti,eih->eth", A, Wd)
    Y = np.einsum("te,eth->th", R, F)
    if p.get("sh_gate") is not None:
        Sg = dequant(p["sh_gate"], p["sh_s_gate"], dt)
        Su = dequant(p["sh_up"], p["sh_s_up"], dt)
        Sd = dequant(p["sh_down"], p["sh_s_down"], dt)
        g, u = X @ Sg, X @ Su
        Y = Y + (g / (1.0 + np.exp(-g)) * u) @ Sd
    return Y


def tiny_problem(dtype="f32", T=12, H=128, I=256, E=5, K=3, seed=0, shared=0, routing=None,
                 routing_kind="uniform"):
    cfg = dict(dtype=dtype, T=T, H=H, I=I, E=E, K=K, routing=routing_kind, shared_inter=shared,
               global_experts=4 * E)
    return inputs.make_problem(cfg, seed=seed, device="cpu", routing=routing)


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---- pins ------------------------------------------------------------------

def pin_dispatch_numpy(lib):
    rng = np.random.default_rng(11)
    cases = []
    for T, K, E in [(1, 1, 1), (7, 3, 5), (64, 2, 8), (333, 8, 128), (50, 8, 256)]:
        ids = rng.integers(-1, E, size=(T, K)).astype(np.int32)  # -1s and duplicates
        cases.append((ids, E))
    cases.append((np.full((9, 4), -1, np.int32), 6))                    # nothing local
    cases.append((np.full((9, 4), 2, np.int32), 6))                     # one hot expert
    cases.append((np.zeros((0, 4), np.int32), 6))                       # empty batch
    ids, _ = inputs.make_routing(512, 128, 8, seed=3, kind="zipf")     # skew, empty experts
    cases.append((ids, 128))
    ids, _ = inputs.make_routing(256, 32, 8, seed=4, kind="local_shard", global_experts=256)
    cases.append((ids, 32))
    for ids, E in cases:
        d = orc.dispatch(ids, E, lib=lib)
        flat = ids.reshape(-1)
        valid = flat >= 0
        counts = np.bincount(flat[valid], minlength=E)
        assert np.array_equal(d["counts"], counts), "counts"
        assert np.array_equal(d["offsets"], np.concatenate([[0], np.cumsum(counts)])), "offsets"
        key = np.where(valid, flat, E)  # invalid slots sort last
        order = np.argsort(key, kind="stable")[: int(valid.sum())]
        assert np.array_equal(d["sorted_assign"], order), "sorted_assign"
        inv = np.full(flat.size, -1)
        inv[order] = np.arange(order.size)
        assert np.array_equal(d["row_of"].reshape(-1), inv), "row_of"


def pin_dispatch_rejects(lib):
    for bad in (-2, 6):
        ids = np.zeros((3, 2), np.int32)
        ids[1, 1] = bad
        try:
            orc.dispatch(ids, 6, lib=lib)
        except ValueError:
            continue
        raise AssertionError("id %d accepted" % bad)


def pin_decoders(lib):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([orc.e4m3_decode(c, lib=lib) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "e4m3 NaN codes"
    assert np.array_equal(got[~nan], ref[~nan]), "e4m3 values"
    bits = np.concatenate([np.arange(0, 65536, 37), [0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x8000]])
    bits = bits[(bits & 0x7F80) != 0x7F80]  # skip inf/NaN
    refb = torch.from_numpy(bits.astype(np.int32)).to(torch.int16).view(torch.bfloat16).double().numpy()
    gotb = np.array([orc.bf16_decode(int(b), lib=lib) for b in bits])
    assert np.array_equal(gotb, refb), "bf16 values"
    refi = codes.view(torch.int8).double().numpy()
    goti = np.array([orc.i8_decode(c, lib=lib) for c in range(256)])
    assert np.array_equal(goti, refi), "int8 values"


def pin_single_expert_dense(lib):
    """E=1, K=1, w=1: the layer is one dense SwiGLU FFN (torch fp64 matmuls)."""
    for dt, H, I in (("f32", 96, 160), ("bf16", 128, 192), ("fp8", 256, 384), ("w8a8", 128, 192)):
        T = 6
        routing = (np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32))
        p = tiny_problem(dt, T=T, H=H, I=I, E=1, K=1, routing=routing)
        x = torch.from_numpy(torch_decode(p["hidden"], dt))
        if dt == "fp8":
            x = x * torch.from_numpy(np.repeat(p["hidden_scales"].double().numpy(), 128, axis=1))
        if dt == "w8a8":
            x = x * p["hidden_scales"].double()[:, None]
        Wg = torch.from_numpy(dequant(p["w_gate"], p["s_gate"], dt)[0])
        Wu = torch.from_numpy(dequant(p["w_up"], p["s_up"], dt)[0])
        Wd = torch.from_numpy(dequant(p["w_down"], p["s_down"], dt)[0])
        ref = (torch.nn.functional.silu(x @ Wg) * (x @ Wu)) @ Wd
        got = orc.forward(p, lib=lib)
        assert rel_err(got, ref.numpy()) < 1e-12, "single expert %s: %g" % (dt, rel_err(got, ref.numpy()))


def pin_brute_force(lib):
    """Random tiny problems, all dtypes, duplicates, -1 slots, shared expert."""
    rng = np.random.default_rng(5)
    for dt, H, I, shared in (("f32", 64, 96, 0), ("bf16", 64, 128, 0), ("fp8", 256, 384, 0),
                             ("f32", 64, 96, 96), ("fp8", 128, 256, 256), ("w8a8", 64, 96, 0),
                             ("w8a8", 64, 96, 160)):
        T, E, K = 10, 4, 3
        ids = rng.integers(-1, E, size=(T, K)).astype(np.int32)
        ids[0] = [1, 1, 1]             # duplicate ids in one row
        ids[1] = [-1, -1, -1]          # token with no local expert
        w = rng.uniform(-0.5, 1.5, size=(T, K)).astype(np.float32)
        p = tiny_problem(dt, T=T, H=H, I=I, E=E, K=K, shared=shared, routing=(ids, w))
        got = orc.forward(p, lib=lib)
        ref = dense_reference(p)
        assert rel_err(got, ref) < 1e-12, "brute force %s shared=%d: %g" % (dt, shared, rel_err(got, ref))
        if not shared:
            assert np.all(got[1] == 0.0), "token without local expert must be exactly 0"


def pin_identical_experts(lib):
    """All experts equal and weights summing to 1: output = dense FFN, any routing."""
    p = tiny_problem("f32", T=16, H=64, I=96, E=6, K=4, seed=2)
    for name in ("w_gate", "w_up", "w_down"):
        p[name] = p[name][:1].expand_as(p[name]).contiguous()
    got = orc.forward(p, lib=lib)
    q = dict(p)
    q["E"], q["K"] = 1, 1
    for name in ("w_gate", "w_up", "w_down"):
        q[name] = p[name][:1].contiguous()
    q["ids"] = torch.zeros((16, 1), dtype=torch.int32)
    q["weights"] = torch.ones((16, 1))
    ref = dense_reference(q)
    assert rel_err(got, ref) < 1e-6, "identical experts: %g" % rel_err(got, ref)  # fp32 weights sum


def pin_permutation(lib):
    p = tiny_problem("bf16", T=20, H=64, I=128, E=5, K=2, seed=4)
    base = orc.forward(p, lib=lib)
    perm = np.random.default_rng(9).permutation(20)
    q = dict(p)
    for k in ("hidden", "ids", "weights"):
        q[k] = p[k][torch.from_numpy(perm)].contiguous()
    got = orc.forward(q, lib=lib)
    assert np.array_equal(got, base[perm]), "token permutation"
    sub = orc.forward(p, tokens=perm[:7], lib=lib)
    assert np.array_equal(sub, base[perm[:7]]), "token subset"


def pin_unused_experts_poisoned(lib):
    rng = np.random.default_rng(6)
    ids = rng.choice(np.array([0, 2, 3, -1], np.int32), size=(9, 2)).astype(np.int32)
    w = rng.uniform(0.1, 1.0, size=(9, 2)).astype(np.float32)
    p = tiny_problem("f32", T=9, H=64, I=96, E=6, K=2, seed=6, routing=(ids, w))
    base = orc.forward(p, lib=lib)
    used = set(p["ids"].numpy().reshape(-1).tolist())
    q = dict(p)
    for name in ("w_gate", "w_up", "w_down"):
        w = p[name].clone()
        for e in range(6):
            if e not in used:
                w[e] = float("nan")
        q[name] = w
    got = orc.forward(q, lib=lib)
    assert len(used) < 6
    assert np.all(np.isfinite(got)) and np.array_equal(got, base), "unused experts leaked"


def pin_linearity(lib):
    p = tiny_problem("f32", T=8, H=64, I=96, E=4, K=2, seed=8)
    base = orc.forward(p, lib=lib)
    q = dict(p)
    q["weights"] = p["weights"] * 0.25  # a power of two: exact in fp32 and fp64
    got = orc.forward(q, lib=lib)
    assert rel_err(got, 0.25 * base) < 1e-15, "linearity in w"
    q["weights"] = torch.zeros_like(p["weights"])
    assert np.all(orc.forward(q, lib=lib) == 0.0), "w = 0"
    q = dict(p)
    ids = p["ids"].clone()
    w = p["weights"].clone()
    ids[:, 1] = -1
    q["ids"] = ids
    r = dict(p)
    w0 = w.clone()
    w0[:, 1] = 0.0
    r["weights"] = w0
    assert rel_err(orc.forward(q, lib=lib), orc.forward(r, lib=lib)) < 1e-15, "-1 equals weight 0"
    z = dict(p)
    z["hidden"] = torch.zeros_like(p["hidden"])
    assert np.all(orc.forward(z, lib=lib) == 0.0), "zero input"


def pin_closed_form(lib):
    with open(os.path.join(GOLDEN, "closed_form_swiglu.json")) as f:
        g = json.load(f)
    p = dict(dtype="f32", hidden=np.array(g["hidden"], np.float32),
             ids=np.array(g["ids"], np.int32), weights=np.array(g["weights"], np.float32),
             w_gate=np.array(g["w_gate"], np.float32), w_up=np.array(g["w_up"], np.float32),
             w_down=np.array(g["w_down"], np.float32), hidden_scales=None, s_gate=None,
             s_up=None, s_down=None)
    got = orc.forward(p, lib=lib)
    assert np.allclose(got, np.array(g["expected"]), rtol=1e-14, atol=1e-15), "closed form %s" % got


ALL_PINS = [pin_dispatch_numpy, pin_dispatch_rejects, pin_decoders, pin_single_expert_dense,
            pin_brute_force, pin_identical_experts, pin_permutation,
            pin_unused_experts_poisoned, pin_linearity, pin_closed_form]
