"""Seeded workload generator (CPU): shapes, routing statistics, FP8 encoding."""
import numpy as np
import torch

from moe_expert_ffn_afd_amd import inputs


def test_routing_uniform_and_reproducible():
    ids, w = inputs.make_routing(256, 128, 8, seed=0)
    ids2, w2 = inputs.make_routing(256, 128, 8, seed=0)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2)
    assert ids.shape == (256, 8) and ids.dtype == np.int32 and w.dtype == np.float32
    assert np.all((ids >= 0) & (ids < 128))
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    assert all(len(set(r)) == 8 for r in ids.tolist())       # top-k picks distinct experts
    assert np.all(np.diff(w, axis=1) <= 0)                   # sorted by probability
    counts = np.bincount(ids.reshape(-1), minlength=128)
    assert counts.min() > 0 and counts.max() < 48             # roughly uniform load


def test_routing_zipf_is_skewed_with_empty_experts():
    ids, w = inputs.make_routing(4096, 128, 8, seed=0, kind="zipf")
    counts = np.bincount(ids.reshape(-1), minlength=128)
    assert (counts == 0).sum() > 0                            # some experts get nothing
    assert counts.max() > 2000                                # one very hot expert
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)


def test_routing_local_shard():
    ids, w = inputs.make_routing(2048, 32, 8, seed=0, kind="local_shard", global_experts=256)
    local = ids >= 0
    assert np.all(ids[local] < 32) and np.all(w[~local] == 0)
    frac = local.mean()
    assert 0.10 < frac < 0.15                                 # about 1/8 of slots are local
    assert np.all(w.sum(1) <= 1.0 + 1e-6)                     # not renormalised after the cut


def test_fp8_rows_and_blocks():
    x = torch.randn(4, 256) * 3
    x[1, :128] = 0.0
    q, s = inputs.quantize_fp8_rows(x)
    assert q.dtype == torch.uint8 and s.shape == (4, 2)
    assert s[1, 0] == 1.0 and torch.all(q[1, :128] == 0)
    amax = x.reshape(4, 2, 128).abs().amax(2)
    assert torch.allclose(s[amax > 0], amax[amax > 0] / 448.0)
    dec = q.view(torch.float8_e4m3fn).float().reshape(4, 2, 128) * s[:, :, None]
    assert torch.all((dec.reshape(4, 256) - x).abs() <= x.abs() * 2 ** -4 + s.repeat_interleave(128, 1) * 2 ** -9)
    w = torch.randn(256, 384) * 0.02
    qw, sw = inputs.quantize_fp8_block(w)
    assert sw.shape == (2, 3)
    assert torch.allclose(sw, w.reshape(2, 128, 3, 128).abs().amax((1, 3)) / 448.0)
    assert qw.view(torch.float8_e4m3fn).float().abs().max() <= 448.0


def test_int8_rows_and_columns():
    x = torch.randn(5, 96) * 3
    x[2] = 0.0
    q, s = inputs.quantize_int8_rows(x)
    assert q.dtype == torch.int8 and s.shape == (5,)
    assert s[2] == 1.0 and torch.all(q[2] == 0)
    amax = x.abs().amax(1)
    assert torch.allclose(s[amax > 0], amax[amax > 0] / 127.0)
    assert q.abs().max() == 127 and torch.all(q.int().abs() <= 127)
    # round to nearest: every value within half a step of its code
    dec = q.float() * s[:, None]
    assert torch.all((dec - x).abs() <= 0.5 * s[:, None] * (1 + 1e-6))
    # the largest element of each row lands exactly on +-127
    assert torch.all(q.gather(1, x.abs().argmax(1, keepdim=True)).abs()[amax > 0] == 127)
    w = torch.randn(200, 48) * 0.02
    w[:, 7] = 0.0
    qw, sw = inputs.quantize_int8_cols(w)
    assert qw.shape == (200, 48) and sw.shape == (48,) and sw[7] == 1.0 and torch.all(qw[:, 7] == 0)
    assert torch.allclose(sw[torch.arange(48) != 7], w.abs().amax(0)[torch.arange(48) != 7] / 127.0)
    assert torch.all((qw.float() * sw[None, :] - w).abs() <= 0.5 * sw[None, :] * (1 + 1e-6))
    # ties go to the even code (torch.round): 2.5 steps -> 2, 3.5 steps -> 4
    qt, st = inputs.quantize_int8_rows(torch.tensor([[127.0, 2.5, 3.5, -2.5]]))
    assert st.item() == 1.0 and qt.tolist() == [[127, 2, 4, -2]]


def test_make_problem_shapes():
    cfg = dict(dtype="fp8", T=8, H=256, I=384, E=3, K=2, routing="uniform", shared_inter=256)
    p = inputs.make_problem(cfg, seed=1)
    assert p["hidden"].shape == (8, 256) and p["hidden_scales"].shape == (8, 2)
    assert p["w_gate"].shape == (3, 256, 384) and p["w_down"].shape == (3, 384, 256)
    assert p["s_gate"].shape == (3, 2, 3) and p["s_down"].shape == (3, 3, 2)
    assert p["sh_gate"].shape == (256, 256) and p["sh_s_down"].shape == (2, 2)
    q = inputs.make_problem(cfg, seed=1)
    assert torch.equal(p["w_up"], q["w_up"]) and torch.equal(p["hidden"], q["hidden"])
    cfg = dict(dtype="w8a8", T=8, H=256, I=384, E=3, K=2, routing="uniform", shared_inter=256)
    p = inputs.make_problem(cfg, seed=1)
    assert p["hidden"].dtype == torch.int8 and p["hidden_scales"].shape == (8,)
    assert p["w_gate"].dtype == torch.int8 and p["s_gate"].shape == (3, 384) and p["s_down"].shape == (3, 256)
    assert p["sh_gate"].shape == (256, 256) and p["sh_s_gate"].shape == (256,) and p["sh_s_down"].shape == (256,)


def test_workload_table():
    for name, cfg in inputs.WORKLOADS.items():
        c = inputs.workload(name)
        assert c["name"] == name and name in inputs.WORKLOAD_TITLES
        if c["dtype"] == "fp8":
            assert c["H"] % 128 == 0 and c["I"] % 128 == 0
