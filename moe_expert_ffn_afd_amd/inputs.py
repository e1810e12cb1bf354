"""Seeded synthetic inputs for the FFN-side MoE layer.

This module is shared by the HIP path's tests and benchmark and by the oracle
tests.  It holds none of the layer's own arithmetic: only the draws that on
the pages happen before the expert GPU sees the data -- top-k routing chosen
on the attention side ("FastAFD" summary, System Design item 1), the token
hidden states, and the expert weights -- plus their 8-bit encodings: block-FP8
(attention GPUs publish FP8 tokens, System Design item 2; experts are kept in
block-FP8, item 1), with torch's own E4M3FN cast, and W8A8 int8 (the expert
precision of the vLLM AFD plugin blog's decode benchmark), with torch's
round-half-to-even.

Workloads (synthetic stand-ins for the pages' models and prompts, which are
not available here; the pages print no layer shapes):

  tiny          fp32, T=64,  H=256,  E=8,   I=512,  top-2, uniform routing
  decode        bf16, T=256, H=4096, E=128, I=1536, top-8, uniform routing
  aggregated    bf16, T=4096, H=4096, E=128, I=1536, top-8, Zipf(1.2) expert
                popularity over a random permutation of the experts
  fp8_shared    block-FP8, T=2048, H=7168, E=256, I=2048, top-8, plus one
                always-on shared expert (I=2048, weight 1)
  verify_shard  block-FP8, 1024 requests x 4 verified tokens = T=4096,
                H=7168, the 32 local experts [0,32) of 256 global ones,
                I=2048, top-8 over the 256 with non-local slots set to -1;
                run as two microbatches of 2048 tokens
  w8a8_shared   W8A8 int8 (per-channel weight scales, per-token activation
                scales), the fp8_shared shape: T=2048, H=7168, E=256, I=2048,
                top-8, plus one shared expert (I=2048)

Hidden ~ N(0,1); weights ~ N(0, 0.02); router logits ~ N(0,1) (+ log Zipf
prior for `aggregated`); softmax, top-k (ties to the lower expert index),
renormalised over the k chosen.  Routing uses numpy's PCG64 seeded with
`seed`; hidden states and weights use a torch generator on the target device
seeded from `seed` (values therefore depend on the device type).
"""
from __future__ import annotations

import numpy as np
import torch

FP8_MAX = 448.0  # largest finite OCP E4M3FN value
FP8_GROUP = 128  # activation group (1 x 128) and weight block (128 x 128) edge
I8_MAX = 127.0   # largest int8 code of the symmetric W8A8 encoding

WORKLOADS = {
    "tiny": dict(dtype="f32", T=64, H=256, E=8, I=512, K=2, routing="uniform"),
    "decode": dict(dtype="bf16", T=256, H=4096, E=128, I=1536, K=8, routing="uniform"),
    "aggregated": dict(dtype="bf16", T=4096, H=4096, E=128, I=1536, K=8, routing="zipf",
                       zipf_s=1.2),
    "fp8_shared": dict(dtype="fp8", T=2048, H=7168, E=256, I=2048, K=8, routing="uniform",
                       shared_inter=2048),
    "verify_shard": dict(dtype="fp8", T=4096, H=7168, E=32, I=2048, K=8, routing="local_shard",
                         global_experts=256, microbatches=2, draft_q=4),
    "w8a8_shared": dict(dtype="w8a8", T=2048, H=7168, E=256, I=2048, K=8, routing="uniform",
                        shared_inter=2048),
}

WORKLOAD_TITLES = {
    "tiny": "tiny_f32_T64_H256_E8_I512_top2",
    "decode": "decode_bf16_T256_H4096_E128_I1536_top8",
    "aggregated": "aggregated_zipf1.2_bf16_T4096_H4096_E128_I1536_top8",
    "fp8_shared": "blockfp8_shared_T2048_H7168_E256+1_I2048_top8",
    "verify_shard": "blockfp8_verify_q4_T4096_H7168_E32of256_I2048_top8_2x2048",
    "w8a8_shared": "w8a8_shared_T2048_H7168_E256+1_I2048_top8",
}


def workload(name: str, **overrides) -> dict:
    cfg = dict(WORKLOADS[name])
    cfg.setdefault("shared_inter", 0)
    cfg.update(overrides)
    cfg["name"] = name
    return cfg


# --------------------------------------------------------------------------
# routing (attention side)
# --------------------------------------------------------------------------

def make_routing(T: int, E: int, K: int, seed: int = 0, kind: str = "uniform",
                 zipf_s: float = 1.2, global_experts: int | None = None):
    """ids int32 [T,K] (ids in [0,E) or -1) and weights fp32 [T,K].

    kind: 'uniform' (iid N(0,1) logits), 'zipf' (N(0,1) + log of a Zipf(s)
    prior over a seeded random permutation of the experts) or 'local_shard'
    (top-K over `global_experts` experts, then slots whose expert lies outside
    the local shard [0,E) become id -1 with weight 0; the remaining weights
    are NOT renormalised, so the output is this shard's partial sum).
    """
    rng = np.random.default_rng(seed)
    n = E
    if kind == "zipf":
        perm = rng.permutation(E)          # perm[j] = expert of popularity rank j+1
        rank = np.empty(E)
        rank[perm] = np.arange(1, E + 1)
        prior = rank ** (-zipf_s)
        logits = rng.standard_normal((T, E)) + np.log(prior / prior.sum())
    elif kind == "local_shard":
        n = int(global_experts)
        logits = rng.standard_normal((T, n))
    elif kind == "uniform":
        logits = rng.standard_normal((T, E))
    else:
        raise ValueError("unknown routing kind %r" % kind)
    if K > n:
        raise ValueError("top-k larger than the expert count")
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    top = np.argsort(-p, axis=1, kind="stable")[:, :K]
    w = np.take_along_axis(p, top, axis=1)
    w = w / w.sum(axis=1, keepdims=True)
    if kind == "local_shard":
        local = top < E
        top = np.where(local, top, -1)
        w = np.where(local, w, 0.0)
    return np.ascontiguousarray(top, dtype=np.int32), np.ascontiguousarray(w, dtype=np.float32)


# --------------------------------------------------------------------------
# block-FP8 encoding (torch's E4M3FN cast, round to nearest even)
# --------------------------------------------------------------------------

def quantize_fp8_rows(x: torch.Tensor):
    """x [T,H] fp32 -> (codes uint8 [T,H], scales fp32 [T,H/128]); one scale per
    1x128 group: amax/448 (1 when the group is all zero)."""
    T, H = x.shape
    g = x.float().reshape(T, H // FP8_GROUP, FP8_GROUP)
    amax = g.abs().amax(dim=2)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (g / scale[:, :, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(T, H).contiguous(), scale.contiguous()


def quantize_fp8_block(w: torch.Tensor):
    """w [R,C] fp32 -> (codes uint8 [R,C], scales fp32 [R/128, C/128]); one scale
    per 128x128 block: amax/448 (1 when the block is all zero)."""
    R, C = w.shape
    b = w.float().reshape(R // FP8_GROUP, FP8_GROUP, C // FP8_GROUP, FP8_GROUP)
    amax = b.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (b / scale[:, None, :, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(R, C).contiguous(), scale.contiguous()


# --------------------------------------------------------------------------
# W8A8 encoding (symmetric int8, round half to even)
# --------------------------------------------------------------------------

def _int8_codes(v: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    return torch.round(v / scale).clamp(-I8_MAX, I8_MAX).to(torch.int8)


def quantize_int8_rows(x: torch.Tensor):
    """x [T,H] fp32 -> (codes int8 [T,H], scales fp32 [T]); one scale per
    token: amax/127 (1 when the row is all zero)."""
    x = x.float()
    amax = x.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / I8_MAX, torch.ones_like(amax))
    return _int8_codes(x, scale[:, None]).contiguous(), scale.contiguous()


def quantize_int8_cols(w: torch.Tensor):
    """w [R,C] fp32 -> (codes int8 [R,C], scales fp32 [C]); one scale per
    output channel (column): amax/127 (1 when the column is all zero)."""
    w = w.float()
    amax = w.abs().amax(dim=0)
    scale = torch.where(amax > 0, amax / I8_MAX, torch.ones_like(amax))
    return _int8_codes(w, scale[None, :]).contiguous(), scale.contiguous()


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------

def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + stream) & 0x7FFFFFFFFFFFFFFF)
    return g


def make_hidden(T: int, H: int, dtype: str, seed: int = 0, device="cpu"):
    """(hidden, hidden_scales or None); hidden ~ N(0,1) before encoding."""
    x = torch.randn((T, H), generator=_gen(device, seed, 1), device=device, dtype=torch.float32)
    if dtype == "f32":
        return x, None
    if dtype == "bf16":
        return x.to(torch.bfloat16), None
    if dtype == "w8a8":
        return quantize_int8_rows(x)
    return quantize_fp8_rows(x)


def make_expert_weights(E: int, H: int, I: int, dtype: str, seed: int = 0, device="cpu",
                        stream: int = 2, std: float = 0.02):
    """Wg, Wu [E,H,I], Wd [E,I,H] ~ N(0, std), encoded; FP8 also returns the
    [E,H/128,I/128], [E,H/128,I/128], [E,I/128,H/128] block scales, W8A8 the
    [E,I], [E,I], [E,H] per-output-channel scales."""
    g = _gen(device, seed, stream)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8, "w8a8": torch.int8}[dtype]
    wg = torch.empty((E, H, I), dtype=tdt, device=device)
    wu = torch.empty((E, H, I), dtype=tdt, device=device)
    wd = torch.empty((E, I, H), dtype=tdt, device=device)
    scales = None
    if dtype == "fp8":
        scales = (torch.empty((E, H // FP8_GROUP, I // FP8_GROUP), device=device),
                  torch.empty((E, H // FP8_GROUP, I // FP8_GROUP), device=device),
                  torch.empty((E, I // FP8_GROUP, H // FP8_GROUP), device=device))
    elif dtype == "w8a8":
        scales = (torch.empty((E, I), device=device), torch.empty((E, I), device=device),
                  torch.empty((E, H), device=device))
    for e in range(E):  # one expert at a time keeps the fp32 staging small
        for j, (dst, shape) in enumerate(((wg, (H, I)), (wu, (H, I)), (wd, (I, H)))):
            w = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
            if dtype in ("fp8", "w8a8"):
                q, s = quantize_fp8_block(w) if dtype == "fp8" else quantize_int8_cols(w)
                dst[e].copy_(q)
                scales[j][e].copy_(s)
            else:
                dst[e].copy_(w.to(tdt))
    return wg, wu, wd, scales


def make_problem(cfg: dict, seed: int = 0, device="cpu", routing=None) -> dict:
    """Full input set for one workload as torch tensors on `device`.

    `routing` = (ids, weights) overrides the drawn routing (adversarial tests).
    Returns a dict with dtype, T, H, I, E, K, hidden, hidden_scales, ids,
    weights, w_gate, w_up, w_down, s_gate, s_up, s_down and, with a shared
    expert, sh_gate, sh_up, sh_down, sh_s_gate, sh_s_up, sh_s_down.
    """
    T, H, I, E, K, dt = cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["K"], cfg["dtype"]
    if routing is None:
        ids, w = make_routing(T, E, K, seed, cfg.get("routing", "uniform"), cfg.get("zipf_s", 1.2),
                              cfg.get("global_experts"))
    else:
        ids, w = (np.ascontiguousarray(a) for a in routing)
    hidden, hscales = make_hidden(T, H, dt, seed, device)
    wg, wu, wd, sc = make_expert_weights(E, H, I, dt, seed, device)
    p = dict(dtype=dt, T=T, H=H, I=I, E=E, K=K, hidden=hidden, hidden_scales=hscales,
             ids=torch.from_numpy(np.asarray(ids, np.int32)).to(device),
             weights=torch.from_numpy(np.asarray(w, np.float32)).to(device),
             w_gate=wg, w_up=wu, w_down=wd,
             s_gate=sc[0] if sc else None, s_up=sc[1] if sc else None, s_down=sc[2] if sc else None)
    Is = cfg.get("shared_inter", 0)
    if Is:
        shg, shu, shd, ssc = make_expert_weights(1, H, Is, dt, seed, device, stream=3)
        p.update(sh_gate=shg[0], sh_up=shu[0], sh_down=shd[0],
                 sh_s_gate=ssc[0][0] if ssc else None, sh_s_up=ssc[1][0] if ssc else None,
                 sh_s_down=ssc[2][0] if ssc else None)
    return p


def slice_tokens(p: dict, t0: int, t1: int) -> dict:
    """The same problem restricted to tokens [t0, t1) (a microbatch)."""
    q = dict(p)
    q["T"] = t1 - t0
    for k in ("hidden", "hidden_scales", "ids", "weights"):
        if q.get(k) is not None:
            q[k] = q[k][t0:t1].contiguous()
    return q


def expected_routed_rows(ids: np.ndarray) -> int:
    return int((np.asarray(ids) >= 0).sum())


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = ["WORKLOADS", "WORKLOAD_TITLES", "workload", "make_routing", "quantize_fp8_rows",
           "quantize_fp8_block", "quantize_int8_rows", "quantize_int8_cols", "I8_MAX", "make_hidden",
           "make_expert_weights", "make_problem",
           "slice_tokens", "FP8_MAX", "FP8_GROUP", "ceil_div", "expected_routed_rows"]
