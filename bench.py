"""Benchmark of the latent-MoE layer forward on one MI355X.

One step = one full layer forward (router GEMM, routing, permutation, down projection,
grouped FC1 + SituGLU, grouped FC2 + combine, shared expert, RMSNorm + up projection
with the shared add) over one batch of seeded synthetic tokens already resident in HBM.

Prints one JSON line: layer tokens/s of the decode-shape layer (T=8, H=7168, L=2048,
E=896, top-16, d=512, shared I=4096, bf16), routing us/call at T=1024, the roofline
fraction of the dominant kernel (grouped FC1 + SituGLU, timed with HIP events on its
launch stream; HBM-bound for the weight-streaming kernels of decode and MX experts,
MFMA-bound for the tiled kernel of prefill) and the CPU oracle timed on a bounded sample
of the same work.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_bf16]
                       [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "latent-MoE layer tokens/sec + route µs/call; % of HBM BW / MFMA peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def layer_bytes(cfg, n_touched):
    """Algorithmic HBM bytes of one layer step: every weight byte of the dense projections,
    the shared expert and the touched experts read once; activations read and written
    once (bf16 = 2 bytes)."""
    e = 2
    dense = e * (cfg.E * cfg.H + cfg.L * cfg.H + 3 * cfg.H * cfg.I + cfg.H * cfg.L)
    experts = n_touched * 3 * cfg.L * cfg.d * (e if cfg.experts != "mx" else 0.5 + 1 / 32)
    acts = e * cfg.T * cfg.H * 2
    return int(dense + experts + acts)


def fc1_bytes(cfg, n_touched, rows):
    """Algorithmic bytes of one grouped FC1 + SituGLU launch: W1 of each touched expert
    (2d x L) read once, the latent rows read once, the activation rows written once.
    bf16: 2 bytes per element; MX: 0.5 byte per e2m1 weight + 1/32 byte of scale, 1 byte
    per e4m3 activation + 1/32 byte of scale."""
    if cfg.experts == "mx":
        w = n_touched * 2 * cfg.d * cfg.L * (0.5 + 1 / 32)
        return int(w + cfg.T * cfg.L * (1 + 1 / 32) + rows * cfg.d * (1 + 1 / 32))
    return n_touched * 2 * cfg.d * cfg.L * 2 + cfg.T * cfg.L * 2 + rows * cfg.d * 2


def fc1_roofline(cfg, n_touched, rows, pairs, fc1_ms):
    """Roofline of the grouped FC1 + SituGLU launch for the workload's kernel: the
    weight-streaming GEMM (decode, MX experts) is bound by HBM, its algorithmic bytes per
    launch from fc1_bytes; the LDS-tiled MFMA GEMM (128-row expert tiles, prefill) is bound
    by the bf16 matrix cores, its algorithmic work 2 * pairs * 2d * L flops (the token-expert
    pairs, not the padded rows it also computes)."""
    if cfg.experts != "mx" and cfg.tile_m == 128:
        flops = 2 * pairs * 2 * cfg.d * cfg.L
        achieved = flops / (fc1_ms * 1e-3) / 1e12
        return {"kernel": "grouped FC1 + SituGLU (tiled_gemm_kernel, 128 x 512 tiles, SituGLU epilogue)",
                "bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops,
                "executed_rows": rows, "avg_ms": round(fc1_ms, 5), "n_touched_experts": n_touched}
    fb = fc1_bytes(cfg, n_touched, rows)
    achieved = fb / (fc1_ms * 1e-3) / 1e9
    kern = ("stream_gemm_mx_kernel, MXFP8 x MXFP4 scaled MFMA" if cfg.experts == "mx"
            else "stream_gemm_kernel, SituGLU epilogue")
    return {"kernel": f"grouped FC1 + SituGLU ({kern})", "bound": "hbm", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": fb, "avg_ms": round(fc1_ms, 5), "n_touched_experts": n_touched}


def fc1_traffic(cfg, seed):
    """HBM bytes per FC1 launch from the workload's committed counter profile
    (profiles/fc1_<workload>_pmc.md: FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of
    known size); None when there is none, for another seed, or when the kernel sources
    changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"fc1_{cfg.name}_pmc.md")
    if seed != 2 or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", " ", "#", "`")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for f in kv["kernel_sources"].split():
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != kv["kernel_sources_sha256"]:
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def route_microbench(torch, B, LI, reps=200):
    """lmoe_route at T=1024, E=896, K=16 (us per call, algorithmic bytes), plus the grouped
    (8 groups, 4 kept) and Renormalize methods on the same logits. The `reps` calls are
    captured in a HIP graph and replayed, so the figure is the GPU's time per call rather
    than the rate at which the host can issue them (about 8-10 us per call from Python)."""
    cfg = LI.ROUTE_MASKED
    logits = LI.make_route_logits(cfg, 3, device="cuda")
    bias = LI.make_bias(cfg, 3, device="cuda")
    ids = torch.empty(cfg.T, cfg.K, dtype=torch.int32, device="cuda")
    w = torch.empty(cfg.T, cfg.K, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    calls = {
        "sigmoid": lambda: B.lmoe_route(cfg.T, cfg.E, cfg.K, logits, bias, cfg.rsf, 1, ids, w),
        "grouped_8_4": lambda: B.lmoe_route_grouped(cfg.T, cfg.E, cfg.K, 8, 4, logits, bias, cfg.rsf, 1, ids, w),
        "renormalize": lambda: B.lmoe_route_renormalize(cfg.T, cfg.E, cfg.K, logits, ids, w),
    }
    us = {}
    for name, call in calls.items():
        for _ in range(20):
            call()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                call()
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        us[name] = a.elapsed_time(b) * 1000.0 / reps
        del graph
    nbytes = cfg.T * cfg.E * 4 + cfg.E * 4 + cfg.T * cfg.K * 8
    return us, nbytes


def cpu_baseline(torch, LI, cfg, seed, X_cpu, n_tokens):
    """The oracle timed on the host on `n_tokens` tokens of the same workload."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import numpy as np

    import oracle
    from gpu_helpers import oracle_weights, run_oracle_layer
    w_cpu = LI.make_layer_weights(cfg, seed, device="cpu", experts=False)
    o = oracle_weights(cfg, seed, w_cpu)
    X64 = X_cpu[:n_tokens].to(torch.float64).numpy()
    # expert weights are generated ahead of the timed region (the oracle reads arrays)
    ids, _, _ = oracle.route(oracle.router_logits(X64, o["W_r"]), o["bias"], cfg.K, cfg.rsf)
    for e in np.unique(ids):
        o["W1"][e], o["W2"][e]
    reps, t0 = 0, time.perf_counter()
    while True:      # repeat the sample until about 10 s of CPU work
        run_oracle_layer(cfg, o, X64)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0:
            break
    return reps * n_tokens / dt, dt, reps


def blas_threads():
    """Threads numpy's BLAS runs the oracle's matrix products on (the host threads it uses)."""
    try:
        from threadpoolctl import threadpool_info
        n = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_bf16")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=8)
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB (fp32 multiply by one) before the "
                         "layer, as the reference kernel for HBM byte counters")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of the layer step instead of eager launches")
    ap.add_argument("--schedule", choices=["one_stream", "shared_stream", "router_stream"], default="shared_stream",
                    help="shared_stream: the shared expert runs on a second stream; router_stream: also the "
                         "router GEMM and routing on a third")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build has no multi-GPU path)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import lmoe_inputs as LI
    from latent_moe_layer_sigmoid_amd import LatentMoELayer, LayerShape, StepTimer
    from latent_moe_layer_sigmoid_amd import binding as B
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    cfg = LI.CONFIGS[args.workload]
    log(f"workload {cfg.name}: generating weights on the GPU")
    w = LI.make_layer_weights(cfg, args.seed, device="cuda")
    shape = LayerShape(H=cfg.H, L=cfg.L, E=cfg.E, K=cfg.K, d=cfg.d, I=cfg.I, dtype=cfg.dtype, experts=cfg.experts,
                       beta=cfg.beta, linear_beta=cfg.linear_beta, rsf=cfg.rsf, eps=cfg.eps, tile_m=cfg.tile_m)
    layer = LatentMoELayer(shape, w, shared_stream=args.schedule == "shared_stream",
                           router_stream=args.schedule == "router_stream")
    X_cpu = LI.make_x(cfg, args.seed)
    X = X_cpu.to("cuda")
    stream = torch.cuda.current_stream()

    if args.calibrate_copy_mb > 0:
        n = args.calibrate_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)      # reads and writes n * 4 bytes
        torch.cuda.synchronize()
        log(f"calibration copy: {n * 4} bytes read, {n * 4} bytes written")
        del src, dst

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        layer.forward(X)
    torch.cuda.synchronize()

    step = (lambda: layer.forward(X))
    if args.graph:
        graph = layer.capture(X)
        step = graph.replay
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()

    # timed region: K whole-layer steps, back to back
    log(f"timing {args.steps} steps ({'graph replays' if args.graph else 'eager launches'})")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1000.0 / args.steps
    tok_s = cfg.T * args.steps / elapsed

    # per-step kernel durations (events on the launch stream), separate pass
    timer = StepTimer(stream)
    for _ in range(args.steps):
        layer.forward(X, timer=timer)
    torch.cuda.synchronize()
    dur = timer.durations()

    b = layer.buffers(cfg.T)
    counts = b["counts"].cpu()
    n_touched = int((counts > 0).sum())
    rows = int(b["tile_offsets"][-1].item())
    fc1_ms = dur["fc1"]
    roof = fc1_roofline(cfg, n_touched, rows, cfg.T * cfg.K, fc1_ms)
    roof["traffic"] = fc1_traffic(cfg, args.seed)
    lb = layer_bytes(cfg, n_touched)
    log(f"n_touched={n_touched} rows={rows} fc1={fc1_ms * 1e3:.1f}us step={ms_per_step * 1e3:.1f}us "
        f"layer bytes={lb / 1e6:.1f}MB")
    log("per-step us: " + ", ".join(f"{k}={v * 1e3:.1f}" for k, v in dur.items()))

    route_all, route_bytes = route_microbench(torch, B, LI)
    route_us = route_all["sigmoid"]
    log("route T=1024 us/call: " + ", ".join(f"{k}={v:.2f}" for k, v in route_all.items()))

    res = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded counter-based generator; random-init weights)",
        "config": {"workload": f"{cfg.name}: T={cfg.T} H={cfg.H} L={cfg.L} E={cfg.E} top-{cfg.K} d={cfg.d} "
                               f"shared I={cfg.I} experts={cfg.experts} tile_m={cfg.tile_m}",
                   "tokens_per_step": cfg.T, "seed": args.seed, "schedule": args.schedule,
                   "launch": "hip_graph" if args.graph else "eager"},
        "roofline": roof,
        "layer_hbm": {"algorithmic_bytes": lb, "achieved_GBs": round(lb / (ms_per_step * 1e-3) / 1e9, 1),
                      "frac": round(lb / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "route_us_per_call": round(route_us, 3),
        "route_hbm_frac": round(route_bytes / (route_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 5),
        "route_other_us_per_call": {k: round(v, 3) for k, v in route_all.items() if k != "sigmoid"},
        "step_us": {k: round(v * 1e3, 2) for k, v in dur.items()},
    }
    if not args.no_cpu_baseline:
        n = min(args.cpu_tokens, cfg.T)
        log(f"cpu baseline: oracle on {n} tokens")
        v, dt, reps = cpu_baseline(torch, LI, cfg, args.seed, X_cpu, n)
        res["cpu_baseline"] = {"value": round(v, 4), "unit": "tokens/s", "cores": blas_threads(),
                               "kind": "oracle",
                               "sample": f"{n} of the {cfg.T} tokens of one step ({n * cfg.K} expert pairs), "
                                         f"repeated {reps}x, numpy float64, {dt:.1f} s"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
