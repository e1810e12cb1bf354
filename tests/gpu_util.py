"""Helpers of the GPU tests: run the HIP layer through the C ABI and compare it
with the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

from moe_expert_ffn_afd_amd import afd, inputs
from oracle import oracle as orc

# max|gpu - oracle| <= TOL * max|oracle| over the compared outputs.  bf16 and
# block-FP8 bounds are the layer's stated accuracy targets; the fp32 bound is
# derived from fp32 rounding of the K = H and K = I dot products (u = 6e-8,
# growth ~ sqrt(K) << 170 u); the W8A8 bound from the per-row int8
# re-quantisation of h on the GPU (half a step, amax/254, with amax about ten
# times h's rms: expected max|err|/max|ref| about 0.03-0.04).
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "w8a8": 6e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_host_problem(p: dict) -> dict:
    return {k: (v.detach().cpu() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}


# canary-guarded buffers: bytes of each workspace band, output elements before
# and after a caller's out inside its guarded tensor, and that tensor's canary
GUARD = 1 << 16
PAD = 1 << 15
CANARY = 0x5A


def guarded_out(layer, T):
    """(buffer, out): out[T, H] inside a larger tensor filled with CANARY bytes."""
    dt = torch.float32 if layer.dtype == "f32" else torch.bfloat16
    buf = torch.empty(T * layer.H + 2 * PAD, dtype=dt, device="cuda")
    buf.view(torch.uint8).fill_(CANARY)
    return buf, buf[PAD:PAD + T * layer.H].view(T, layer.H)


def check_out_guard(buf, T, H):
    b = buf.view(torch.uint8)
    esz = buf.element_size()
    head, tail = b[:PAD * esz], b[(PAD + T * H) * esz:]
    assert bool((head == CANARY).all()), "bytes before out[0, 0] were written"
    assert bool((tail == CANARY).all()), "bytes after out[T-1, H-1] were written"


def run_layer_guarded(p: dict):
    """The forward on a handle with canary bands, into a guarded output; asserts
    that no band byte (workspace or output) was written."""
    layer = afd.Layer(p)
    layer.set_canaries(GUARD)
    buf, out = guarded_out(layer, p["T"])
    layer.forward(p["hidden"], p["hidden_scales"], p["ids"], p["weights"], out=out)
    torch.cuda.synchronize()
    check_out_guard(buf, p["T"], p["H"])
    assert layer.check_canaries() == 0
    return layer, out


def run_layer(p: dict, layer=None, stream=None, max_tokens=None):
    layer = layer or afd.Layer(p, max_tokens=max_tokens)
    out = layer.forward(p["hidden"], p["hidden_scales"], p["ids"], p["weights"], stream=stream)
    torch.cuda.synchronize()
    return layer, out


# the oracle's threads: the host cores this process may use, at most 16 (a GPU
# box's share of its host)
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_out(p_host: dict, tokens=None):
    return orc.forward(p_host, tokens=tokens, nthreads=ORACLE_THREADS)


def compare(gpu_out: torch.Tensor, ref: np.ndarray, dtype: str, tokens=None, what=""):
    g = gpu_out.float().cpu().numpy().astype(np.float64)
    if tokens is not None:
        g = g[tokens]
    assert np.all(np.isfinite(g)), "non-finite GPU output " + what
    err = float(np.max(np.abs(g - ref))) if ref.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    say("  %s max|err| = %.3e, max|ref| = %.3e, ratio = %.3e (tol %.0e)" %
        (what, err, scale, err / scale if scale else 0.0, TOL[dtype]))
    assert err <= TOL[dtype] * scale, "%s: max|err| %.3e > %.0e * max|ref| %.3e" % (what, err, TOL[dtype], scale)
    return err / scale if scale else 0.0


def check_dispatch(layer, p: dict):
    T = p["T"]
    got = layer.dispatch(T)
    want = orc.dispatch(p["ids"].cpu().numpy(), p["E"])
    for k in ("counts", "offsets", "sorted_assign", "row_of"):
        assert np.array_equal(got[k], want[k]), "dispatch %s differs" % k
    return want


def problem(cfg: dict, seed=0, routing=None):
    return inputs.make_problem(cfg, seed=seed, device="cuda", routing=routing)


# ---------------------------------------------------------------------------
# m-tiles of a batch, for choosing compared tokens
# ---------------------------------------------------------------------------

def tile_lists(dtype: str, T: int, E: int, K: int, counts, shared: bool):
    """The library's two m-tile lists for a batch, from the oracle's per-expert
    counts and the tile policy the library documents (include/afd_ffn.h,
    api.hip): fp32 has one list of 32-row tiles.  Otherwise light tiles hold
    32*mr rows (mr = 1 up to 32 routed rows per expert on average, else 2) and
    experts with more rows go to the heavy list (256-row bf16 tiles, 128-row
    block-FP8 and W8A8 tiles), the shared expert too once T exceeds a light
    tile.  bf16
    batches with no shared expert and at most 32 rows per expert on average keep
    every expert light (tiles of 32, or of 64 past 16 rows per expert on
    average) unless the largest expert exceeds two such tiles.  Block-FP8
    and W8A8 batches of at least 128 routed rows per expert on average put
    the experts of more than 128 rows (the shared expert too) in a third,
    tiled list of 256-row tiles.
    Returns {"light": [...], "heavy": [...], "tiled": [...]}, each tile
    (expert, first row in the expert, rows); the shared expert is expert E, its
    rows are tokens."""
    counts = np.asarray(counts)
    n_flat = T * K
    if dtype == "f32":
        bm, bm_heavy, heavy_min = 32, 32, 1 << 30
    else:
        mr = 1 if n_flat <= 32 * E else 2
        bm = 32 * mr
        bm_heavy = 128 if dtype in ("fp8", "w8a8") else 256
        heavy_min = bm + 1
        if dtype == "bf16" and not shared and n_flat <= 32 * E:
            mr_lo = 1 if n_flat <= 16 * E else 2
            if counts.max(initial=0) < 2 * 32 * mr_lo + 1:
                bm, heavy_min = 32 * mr_lo, 1 << 30
    tiled_min = 129 if dtype in ("fp8", "w8a8") and n_flat >= 128 * E else 1 << 30
    lists = {"light": [], "heavy": [], "tiled": []}
    sizes = list(enumerate(counts.tolist())) + ([(E, T)] if shared else [])
    for e, n in sizes:
        kind = "tiled" if n >= tiled_min else "heavy" if n >= heavy_min else "light"
        b = {"tiled": 256, "heavy": bm_heavy, "light": bm}[kind]
        for r0 in range(0, n, b):
            lists[kind].append((e, r0, min(b, n - r0)))
    return lists


def tile_covering_tokens(dtype: str, T: int, E: int, K: int, ids, shared: bool, max_tiles=None, seed=0):
    """Tokens whose rows include the first and the last row of every m-tile of
    both lists (of up to max_tiles tiles per list, chosen at random, when
    given), and how many tiles of each list that covers."""
    d = orc.dispatch(np.asarray(ids), E)
    lists = tile_lists(dtype, T, E, K, d["counts"], shared)
    rng = np.random.default_rng(seed)
    tokens, covered = set(), {}
    for name, tiles in lists.items():
        if max_tiles is not None and len(tiles) > max_tiles:
            tiles = [tiles[i] for i in sorted(rng.choice(len(tiles), max_tiles, replace=False))]
        for e, r0, n in tiles:
            for r in (r0, r0 + n - 1):
                tokens.add(r if e == E else int(d["sorted_assign"][d["offsets"][e] + r]) // K)
        covered[name] = (len(tiles), len(lists[name]))
    return np.array(sorted(tokens), dtype=np.int64), covered
