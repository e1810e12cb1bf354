"""Benchmark of the FFN-side MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fp8_shared]

A step is one forward of the whole layer (dispatch count+scan, scatter,
grouped GEMM gate/up + SwiGLU, grouped GEMM down, combine) over one batch of
seeded synthetic tokens already resident in HBM; the verify_shard workload
runs its two microbatches on two streams per step.  The default workload is
the largest one-GPU configuration: block-FP8 experts with a shared expert,
T=2048, H=7168, E=256, I=2048, top-8.  Prints one JSON line with
routed tokens/s, the roofline of the dominant kernel (timed with HIP events
on its own stream inside the timed region, the only stage timed there) and
the oracle's CPU baseline; the per-stage breakdown comes from up to 20 further
steps with every stage timed.  The oracle's sample also checks the measured
run ("check": the sampled tokens' outputs within the stated tolerance, every
microbatch's dispatch bit for bit); the run exits nonzero if that fails.

Other modes: --copy-calibration runs a plain device copy of known size (the
reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters);
--mfma-ceiling measures the MFMA rate sustained with no memory traffic and
the shader clock meanwhile (the ceiling of the MFMA fractions), and the bf16
rate of the LDS-tiled GEMM's inner loop with and without its LDS fragment
reads;
--no-cpu-baseline skips the oracle timing; --graph also times the step
captured in a HIP graph and replayed; --sweep times the layer at the
workload's shape over a range of batch sizes T (the FFN-side time T_e as a
function of the aggregated batch, the term the AFD performance model of
"Revisiting Disaggregated Large Language Model Serving" balances against the
attention side) and prints one JSON line per T.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "f32": 157.3, "w8a8": 5033.2}  # w8a8: dense int8 TOP/s
METRIC = "routed tokens/s per MoE layer on 1 MI355X; % of MFMA/HBM roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
GATE_UP_STAGE = 2  # stage index of the grouped GEMM gate/up + SwiGLU in the library's timing
STAGE_STEPS = 20   # steps with every stage timed, after the timed steps, for the per-stage breakdown
KERNEL_SOURCES = ("gemm.hip", "gemm_stream.h", "gemm_tiled.hip", "gemm_tiled.h", "gemm_ring.hip", "gemm_ring.h",
                  "gemm_tiled8.h",
                  "quant.hip", "quant.h", "fused.h", "fused.hip", "fused_bf16.hip", "combine.h", "afd_device.h",
                  "afd_internal.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "moe_expert_ffn_afd_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def gate_up_kernels(cfg: dict, t_mb: int) -> str:
    """Which launches make up the timed gate/up + SwiGLU stage (the library's tile policy)."""
    if cfg["dtype"] == "fp8":
        return "gate/up + SwiGLU stage: gemm_ring_kernel<true> (heavy and light tiles in one launch)"
    if cfg["dtype"] == "w8a8":
        return ("gate/up + SwiGLU stage: gemm_ring_kernel<true, int8> (heavy and light tiles in one launch), "
                "then quant_rows_kernel (h to int8 per row)")
    if cfg["dtype"] == "f32":
        return "gate/up + SwiGLU stage: gemm_f32_kernel<true> (one launch)"
    if not cfg.get("shared_inter") and t_mb * cfg["K"] <= 32 * cfg["E"]:
        mr = 1 if t_mb * cfg["K"] <= 16 * cfg["E"] else 2
        return ("gate/up + SwiGLU stage: gemm_grouped_kernel<true, %d> (every expert in %d-row tiles) while "
                "the largest expert has at most %d rows, else gemm_mixed_kernel<true, 1>; the dispatch "
                "chooses and the other launch returns at once" % (mr, 32 * mr, 64 * mr))
    mr = 1 if t_mb * cfg["K"] <= 32 * cfg["E"] else 2
    return ("gate/up + SwiGLU stage: gemm_mixed_kernel<true, %d> (one launch: heavy tiles and light "
            "experts on disjoint CUs, side by side)" % mr)


def algorithmic_units(cfg: dict, ids) -> dict:
    """Bytes and flops each kernel must move / do at minimum for this routing."""
    import numpy as np

    T, H, I, E, K = cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["K"]
    dt = cfg["dtype"]
    bw = {"f32": 4, "bf16": 2, "fp8": 1, "w8a8": 1}[dt]
    by = 4 if dt == "f32" else 2
    Is = cfg.get("shared_inter") or 0  # the shared expert's width (0: none)
    ids = np.asarray(ids)
    counts = np.bincount(ids[ids >= 0].reshape(-1), minlength=E)
    N = int(counts.sum())
    S = 1 if Is else 0
    Ns = N + S * T
    ne = int((counts > 0).sum()) + S
    # routed experts' and the shared expert's intermediate widths summed over
    # rows (h elements) and over non-empty experts (weight columns)
    h_elems = N * I + T * Is
    w_cols = (ne - S) * I + Is
    # scales per weight and per activation element: block-FP8 one per 128 x 128
    # weights and per 1 x 128 activations; W8A8 one per output channel (gate/up:
    # per column of H weights, down: per column of I) and per token row
    sc_gu = sc_dn = 4.0 / (128 * 128) if dt == "fp8" else 0.0
    xs = hs = 4.0 / 128 if dt == "fp8" else 0.0
    if dt == "w8a8":
        sc_gu, sc_dn, xs, hs = 4.0 / H, 4.0 / I, 4.0 / H, 4.0 / I
    gu_bytes = w_cols * 2 * H * (bw + sc_gu) + T * H * (bw + xs) + h_elems * (bw + hs)
    dn_bytes = w_cols * H * (bw + sc_dn) + h_elems * (bw + hs) + Ns * H * by
    layer_bytes = (w_cols * H * (2 * (bw + sc_gu) + bw + sc_dn) + T * H * (bw + xs) + T * H * by + T * K * 8)
    return dict(N=N, Ns=Ns, nonempty=ne, gu_bytes=gu_bytes, dn_bytes=dn_bytes, layer_bytes=layer_bytes,
                gu_flops=4.0 * H * h_elems, dn_flops=2.0 * H * h_elems, layer_flops=6.0 * H * h_elems)


def cpu_baseline(p: dict, cfg: dict, budget_s: float = 12.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same batch.
    Returns the baseline record and the oracle's outputs of the sampled tokens
    (the first n of the batch, [n, H] fp64)."""
    import numpy as np
    import torch

    from oracle import oracle as orc

    cores = min(16, len(os.sched_getaffinity(0)))
    host = {k: (v.detach().cpu() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    T = cfg["T"]
    n = min(T, cores)
    t0 = time.perf_counter()
    refs = [orc.forward(host, tokens=np.arange(n, dtype=np.int32), nthreads=cores)]
    t1 = time.perf_counter() - t0
    total_t, total_n = t1, n
    if t1 < budget_s and n < T:
        n2 = int(min(T - n, max(cores, (budget_s - t1) / max(t1, 1e-3) * n)))
        n2 = max(cores, n2 // cores * cores) if n2 >= cores else n2
        t0 = time.perf_counter()
        refs.append(orc.forward(host, tokens=np.arange(n, n + n2, dtype=np.int32), nthreads=cores))
        total_t += time.perf_counter() - t0
        total_n += n2
    rec = {"value": total_n / total_t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": "first %d of the %d tokens of the same seeded batch, fp64, %.1f s" % (total_n, T, total_t),
           "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}
    return rec, np.concatenate(refs, axis=0)


def cpu_model() -> str:
    """The host CPU's model name (first processor of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# stated accuracy of the layer against the fp64 oracle: max|out - ref| <= tol * max|ref|
CHECK_TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "w8a8": 6e-2}


def check_run(cfg: dict, out, ref, layers, parts) -> dict:
    """The timed run's own outputs on the oracle's sampled tokens, and every
    microbatch's dispatch against the oracle's, bit for bit."""
    import numpy as np

    from oracle import oracle as orc

    n = ref.shape[0]
    got = out[:n].double().cpu().numpy()
    err = float(np.max(np.abs(got - ref))) if n else 0.0
    scale = float(np.max(np.abs(ref))) if n else 0.0
    ratio = err / scale if scale else 0.0
    exact = True
    for layer, q in zip(layers, parts):
        d = layer.dispatch(q["T"])
        want = orc.dispatch(q["ids"].cpu().numpy(), cfg["E"])
        exact = exact and all(np.array_equal(d[k], want[k]) for k in ("counts", "offsets", "sorted_assign", "row_of"))
    tol = CHECK_TOL[cfg["dtype"]]
    finite = bool(np.isfinite(got).all())
    return {"tokens": n, "max_err_over_max_ref": float("%.4g" % ratio), "tol": tol, "dispatch_exact": exact,
            "ok": bool(exact and finite and ratio <= tol)}


SWEEP_TOKENS = (64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384)


def sweep_setup(workload: str, seed: int):
    """The sweep's batch sizes, its one seeded batch of the largest size and one
    handle sized for it (each T of the sweep runs the first T tokens)."""
    from moe_expert_ffn_afd_amd import afd, inputs

    base = inputs.workload(workload)
    if base.get("microbatches", 1) != 1:
        sys.exit("--sweep takes a one-microbatch workload")
    H, K = base["H"], base["K"]
    out_row = 4 if base["dtype"] == "f32" else 2
    rows_per_token = K + (1 if base.get("shared_inter") else 0)
    # down outputs [rows, H] stay within 32-bit buffer offsets
    sizes = [t for t in SWEEP_TOKENS if t * rows_per_token * H * out_row < (1 << 31)]
    cfg = dict(base, T=max(sizes))
    p = inputs.make_problem(cfg, seed=seed, device="cuda")
    layer = afd.Layer(p, max_tokens=cfg["T"])
    return cfg, sizes, p, layer


def sweep(args) -> None:
    """Layer time against the batch size at one workload's shape: one handle
    sized for the largest T, one seeded batch of that size, and each T taking
    its first T tokens (the routing's distribution does not change with T)."""
    import torch

    from moe_expert_ffn_afd_amd import inputs

    cfg, sizes, p, layer = sweep_setup(args.workload, args.seed)
    ids_np = p["ids"].cpu().numpy()
    stream = torch.cuda.current_stream()
    for T in sizes:
        q = inputs.slice_tokens(p, 0, T)
        out = layer.out_like(T)
        units = algorithmic_units(dict(cfg, T=T), ids_np[:T])
        for _ in range(args.warmup):
            layer.forward(q["hidden"], q["hidden_scales"], q["ids"], q["weights"], out=out, stream=stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            layer.forward(q["hidden"], q["hidden_scales"], q["ids"], q["weights"], out=out, stream=stream)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / args.steps
        dt = cfg["dtype"]
        print(json.dumps({
            "sweep": inputs.WORKLOAD_TITLES[args.workload], "T": T, "routed_rows": units["N"],
            "nonempty_experts": units["nonempty"], "ms_per_step": round(sec * 1e3, 4),
            "tokens_per_s": round(T / sec, 1), "hbm_gbs": round(units["layer_bytes"] / sec / 1e9, 1),
            "tflops": round(units["layer_flops"] / sec / 1e12, 2),
            "roofline_frac": round(max(units["layer_flops"] / (PEAK_TFLOPS[dt] * 1e12),
                                       units["layer_bytes"] / (PEAK_HBM_GBS * 1e9)) / sec, 4),
            "steps": args.steps, "warmup": args.warmup}), flush=True)
    layer.close()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="fp8_shared",
                    choices=["tiny", "decode", "aggregated", "fp8_shared", "verify_shard", "w8a8_shared"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="the MFMA rate sustained with no memory traffic (bf16, fp8, int8) and its shader clock")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed (graph_ms_per_step)")
    ap.add_argument("--sweep", action="store_true",
                    help="time the layer at the workload's shape for T = 64 ... 16384 (one JSON line per T)")
    ap.add_argument("--fused", action="store_true",
                    help="bf16 / block-FP8 / W8A8 workloads: each forward as one persistent launch (afd_ffn_set_fused)")
    ap.add_argument("--serial", action="store_true",
                    help="microbatch workloads: run the microbatches one after the other on one stream, "
                         "each on every CU (the baseline the two-stream ping-pong is compared with)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer is built for one MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    if args.sweep:
        sweep(args)
        return
    if args.mfma_ceiling:
        from moe_expert_ffn_afd_amd import afd

        res = {}
        for dt, spec in (("bf16", PEAK_TFLOPS["bf16"]), ("fp8", PEAK_TFLOPS["fp8"]), ("w8a8", PEAK_TFLOPS["w8a8"])):
            tf, ghz = afd.afd_ffn_mfma_peak(dt)
            res[dt] = {"tflops": round(tf, 1), "clock_ghz": round(ghz, 3), "frac_of_spec": round(tf / spec, 4)}
        for name, reads in (("bf16_tile_loop_fragments_in_registers", 0), ("bf16_tile_loop_with_lds_reads", 6)):
            tf, ghz = afd.afd_ffn_mfma_lds_peak(reads)
            res[name] = {"tflops": round(tf, 1), "clock_ghz": round(ghz, 3),
                         "frac_of_spec": round(tf / PEAK_TFLOPS["bf16"], 4)}
        print(json.dumps({"mfma_ceiling": res, "note": "8 waves per CU, no memory traffic; bf16_tile_loop_*: the "
                          "LDS-tiled GEMM's 8 MFMAs per 16-deep k slice, with its 6 LDS fragment reads or without"}))
        return
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return

    from moe_expert_ffn_afd_amd import afd, inputs

    cfg = inputs.workload(args.workload)
    p = inputs.make_problem(cfg, seed=args.seed, device="cuda")
    T = cfg["T"]
    mbs = cfg.get("microbatches", 1)
    # each microbatch is its own layer call and reads the weights of its own
    # non-empty experts: the step's units are the sum over microbatches
    ids_np = p["ids"].cpu().numpy()
    mb_cfg = dict(cfg, T=T // mbs)
    per_mb = [algorithmic_units(mb_cfg, ids_np[i * (T // mbs):(i + 1) * (T // mbs)]) for i in range(mbs)]
    units = {k: sum(u[k] for u in per_mb) for k in per_mb[0]}

    layers = [afd.Layer(p, max_tokens=T // mbs)]
    while len(layers) < mbs:
        layers.append(layers[0].clone())
    serial = args.serial and mbs > 1
    for layer in layers:  # the microbatches run side by side, each on its share of the CUs
        layer.set_concurrency(1 if serial else mbs)
        if args.fused:
            layer.set_fused(True)
    if mbs == 1:
        parts = [p]
        streams = [torch.cuda.current_stream()]
    else:
        step = T // mbs
        parts = [inputs.slice_tokens(p, i * step, (i + 1) * step) for i in range(mbs)]
        streams = [torch.cuda.current_stream()] * mbs if serial else [torch.cuda.Stream() for _ in range(mbs)]
    outs = [layers[i].out_like(parts[i]["T"]) for i in range(mbs)]

    def step_fn():
        # the caller's current stream: the default one, or a graph's capture stream
        main_stream = torch.cuda.current_stream()
        if mbs == 1 or serial:  # one stream
            for i in range(mbs):
                q = parts[i]
                layers[i].forward(q["hidden"], q["hidden_scales"], q["ids"], q["weights"], out=outs[i],
                                  stream=main_stream)
            return
        ev = torch.cuda.Event()
        ev.record(main_stream)
        for i in range(mbs):
            streams[i].wait_event(ev)
            q = parts[i]
            layers[i].forward(q["hidden"], q["hidden_scales"], q["ids"], q["weights"], out=outs[i],
                              stream=streams[i])
        for i in range(mbs):
            done = torch.cuda.Event()
            done.record(streams[i])
            main_stream.wait_event(done)

    def collect():
        # average duration per forward of each timed stage (ms), then reset
        tot, nfwd = [0.0] * afd.AFD_NUM_STAGES, 0
        for layer in layers:
            ms, n = afd.afd_ffn_get_timing(layer.handle)
            tot = [a + b for a, b in zip(tot, ms)]
            nfwd += n
        return [m / max(nfwd, 1) for m in tot]

    for _ in range(args.warmup):
        step_fn()
    torch.cuda.synchronize()
    # In the timed steps only the gate/up stage (the roofline's kernel) is
    # bracketed by HIP events on its stream: every event costs the stream a
    # few microseconds, which the step time should not carry.
    for layer in layers:
        afd.afd_ffn_set_timing_stages(layer.handle, [GATE_UP_STAGE])
        afd.afd_ffn_get_timing(layer.handle)  # reset

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_fn()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gu_launch_ms = collect()[GATE_UP_STAGE]

    # The per-stage breakdown comes from further steps with every stage timed.
    for layer in layers:
        afd.afd_ffn_set_timing(layer.handle, True)
    for _ in range(min(args.steps, STAGE_STEPS)):
        step_fn()
    torch.cuda.synchronize()
    per_launch = collect()
    for layer in layers:
        afd.afd_ffn_set_timing(layer.handle, False)

    graph_ms = None
    if args.graph:
        # the same step captured once in a HIP graph (the microbatch streams
        # fork from and join the capture stream) and replayed
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step_fn()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        del graph

    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T / (ms_per_step * 1e-3)
    dt = cfg["dtype"]
    # dominant kernel: grouped GEMM gate/up + SwiGLU (two thirds of the weight bytes and flops)
    gu_launch_s = gu_launch_ms * 1e-3
    launches_per_step = mbs
    # the timed kernel: the gate/up stage, or with --fused the one launch of the whole layer
    gu_bytes = units["layer_bytes" if args.fused else "gu_bytes"] / launches_per_step
    gu_flops = units["layer_flops" if args.fused else "gu_flops"] / launches_per_step
    hbm_ach = gu_bytes / gu_launch_s / 1e9
    mfma_ach = gu_flops / gu_launch_s / 1e12
    # the bound follows the layer's arithmetic intensity against the ridge
    ai = units["layer_flops"] / units["layer_bytes"]
    ridge = PEAK_TFLOPS[dt] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": round(hbm_ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(hbm_ach / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(mfma_ach, 1), "peak": PEAK_TFLOPS[dt], "unit": "TFLOP/s",
                "frac": round(mfma_ach / PEAK_TFLOPS[dt], 4)}
    # both fractions of the same launch, whichever bound the layer sits at
    roof["hbm_frac"] = round(hbm_ach / PEAK_HBM_GBS, 4)
    roof["mfma_frac"] = round(mfma_ach / PEAK_TFLOPS[dt], 4)
    roof["kernel"] = (("the whole layer: %s (one persistent launch per forward)"
                       % ("fused_bf16_kernel" if dt == "bf16" else "fused_kernel")) if args.fused
                      else gate_up_kernels(cfg, T // mbs))
    roof["launch_ms"] = round(gu_launch_ms, 4)
    # launches of this kernel running at once, each on its share of the CUs
    roof["concurrent_launches"] = 1 if serial else mbs
    if not serial and mbs > 1:
        # the concurrent launches start together on disjoint CU shares: their
        # bytes together over their mean duration (the window they share)
        agg = units["layer_bytes" if args.fused else "gu_bytes"] / gu_launch_s / 1e9
        roof["aggregate_hbm_gbs"] = round(agg, 1)
        roof["aggregate_hbm_frac"] = round(agg / PEAK_HBM_GBS, 4)
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f).get(args.workload + ("_fused" if args.fused else ""))
        if tr and tr.get("kernel_hash") == kernel_source_hash():
            traffic = tr.get("bytes_per_launch")
    except (OSError, ValueError):
        pass
    roof["traffic"] = traffic

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8_e4m3_block128", "f32": "f32", "w8a8": "int8_w8a8"}[dt],
        "data": "synthetic (seeded; random-init expert weights N(0,0.02), hidden N(0,1))",
        "config": {"workload": inputs.WORKLOAD_TITLES[args.workload] + ("_fused" if args.fused else ""),
                   "T": T, "H": cfg["H"], "I": cfg["I"],
                   "E": cfg["E"], "top_k": cfg["K"], "shared_inter": cfg.get("shared_inter", 0),
                   "routing": cfg["routing"], "microbatches": mbs, "microbatch_streams": 1 if serial else mbs,
                   "routed_rows": units["N"],
                   "nonempty_experts": units["nonempty"] if mbs == 1 else [u["nonempty"] for u in per_mb],
                   "seed": args.seed},
        "layer": {"assignments_per_s": round(units["N"] / (ms_per_step * 1e-3), 1),  # routed (token, expert) rows
                  "tflops": round(units["layer_flops"] / (ms_per_step * 1e-3) / 1e12, 2),
                  "hbm_gbs": round(units["layer_bytes"] / (ms_per_step * 1e-3) / 1e9, 1),
                  "roofline_frac": round(max(units["layer_flops"] / (PEAK_TFLOPS[dt] * 1e12),
                                             units["layer_bytes"] / (PEAK_HBM_GBS * 1e9)) /
                                         (ms_per_step * 1e-3), 4),
                  "stage_ms": {n: round(v, 4) for n, v in zip(afd.STAGE_NAMES, per_launch)},
                  "stage_ms_steps": min(args.steps, STAGE_STEPS)},
        "roofline": roof,
    }
    if graph_ms is not None:
        result["graph_ms_per_step"] = round(graph_ms, 4)
    ok = True
    if not args.no_cpu_baseline:
        result["cpu_baseline"], ref = cpu_baseline(p, cfg)
        # the oracle's sample doubles as a check of the measured run's outputs
        torch.cuda.synchronize()
        result["check"] = check_run(cfg, torch.cat(outs) if mbs > 1 else outs[0], ref, layers, parts)
        ok = result["check"]["ok"]
    print(json.dumps(result), flush=True)
    for layer in layers[::-1]:
        layer.close()
    if not ok:
        sys.exit("the measured run's outputs or dispatch disagree with the oracle")


if __name__ == "__main__":
    main()
