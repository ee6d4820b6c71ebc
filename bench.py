"""Benchmark of the latent-MoE layer forward on one MI355X.

One step = one full layer forward (router GEMM, routing, permutation, down projection,
grouped FC1 + SituGLU, grouped FC2 + combine, shared expert, RMSNorm + up projection
with the shared add) over one batch of seeded synthetic tokens already resident in HBM.

Prints one JSON line. The headline (`value`) is layer tokens/s of the prefill-shape layer
(T=8192, H=7168, L=2048, E=896, top-16, d=512, shared I=4096, bf16, skewed routing): the
largest workload that one GPU runs. `roofline` is its dominant routed kernel, the grouped
FC1 + SituGLU launch, timed with HIP events on its launch stream: MFMA-bound for the tiled
prefill kernel (and its fraction of the per-expert max(MFMA, HBM) floor), HBM-bound for the
weight-streaming kernels of decode and MX experts. `cpu_baseline` is the CPU oracle on a
bounded sample of the same workload. `workloads` carries the other measurements in the
same run: the decode layer (warm: back-to-back steps on one input; cold: a 1 GiB scratch
write before every step and four inputs in rotation, the flush outside the timed events),
the decode step's time per launch mode (the Python call sequence, the library's own step
lmoe_layer_forward, its HIP graph, torch's HIP graph), the MX-expert layer (warm and cold),
routing us/call at T=1024 (three methods), the masked
SituGLU over the [896, 64, 1024] buffer, the permutation, step-time percentiles, the GPU
clock and a measured device-copy bandwidth.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_bf16]
                       [--no-cpu-baseline] [--no-extras]
"""
import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "latent-MoE layer tokens/sec + route µs/call; % of HBM BW / MFMA peak"
FLUSH_BYTES = 1 << 30        # cold steps: this many bytes written between steps (the MALL is 256 MB)


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


def layer_flops(cfg):
    """Algorithmic flops of one layer step: the dense projections (router, down, shared
    FC1 and FC2, up) over all tokens, and the routed FC1 + FC2 over the T*K token-expert
    pairs."""
    dense = 2 * cfg.T * (cfg.E * cfg.H + cfg.L * cfg.H + 3 * cfg.H * cfg.I + cfg.H * cfg.L)
    routed = 2 * cfg.T * cfg.K * 3 * cfg.L * cfg.d
    return dense + routed


def fc1_bytes(cfg, n_touched, rows):
    """Algorithmic bytes of one grouped FC1 + SituGLU launch: W1 of each touched expert
    (2d x L) read once, the latent rows read once, the activation rows written once.
    bf16: 2 bytes per element; MX: 0.5 byte per e2m1 weight + 1/32 byte of scale, 1 byte
    per e4m3 activation + 1/32 byte of scale."""
    if cfg.experts == "mx":
        w = n_touched * 2 * cfg.d * cfg.L * (0.5 + 1 / 32)
        return int(w + cfg.T * cfg.L * (1 + 1 / 32) + rows * cfg.d * (1 + 1 / 32))
    return n_touched * 2 * cfg.d * cfg.L * 2 + cfg.T * cfg.L * 2 + rows * cfg.d * 2


def fc1_expert_floor_ms(cfg, counts):
    """Per-expert floor of the grouped FC1 launch: for each touched expert, the larger of
    its MFMA time (2 * rows * 2d * L flops at the bf16 peak) and its HBM time (its W1 once,
    its latent rows read and its activation rows written, at 8 TB/s), summed over the
    experts."""
    t = 0.0
    for c in counts:
        if c <= 0:
            continue
        flops = 2.0 * c * 2 * cfg.d * cfg.L
        nbytes = 2.0 * cfg.d * cfg.L * 2 + c * cfg.L * 2 + c * cfg.d * 2
        t += max(flops / (MFMA_BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBS * 1e9))
    return t * 1e3


def fc1_roofline(cfg, n_touched, rows, pairs, fc1_ms, counts=None):
    """Roofline of the grouped FC1 + SituGLU launch for the workload's kernel: the
    weight-streaming GEMM (decode, MX experts) is bound by HBM, its algorithmic bytes per
    launch from fc1_bytes; the LDS-tiled MFMA GEMM (128-row expert tiles, prefill) is bound
    by the bf16 matrix cores, its algorithmic work 2 * pairs * 2d * L flops (the token-expert
    pairs, not the padded rows it also computes); with the expert histogram it also
    reports the launch's fraction of the per-expert max(MFMA, HBM) floor."""
    if cfg.experts != "mx" and cfg.tile_m == 128:
        flops = 2 * pairs * 2 * cfg.d * cfg.L
        achieved = flops / (fc1_ms * 1e-3) / 1e12
        r = {"kernel": "grouped FC1 + SituGLU (tiled_gemm_kernel, 128 x 512 tiles, SituGLU epilogue)",
             "bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops,
             "executed_rows": rows, "avg_ms": round(fc1_ms, 5), "n_touched_experts": n_touched}
        if counts is not None:
            floor = fc1_expert_floor_ms(cfg, counts)
            r["expert_floor_ms"] = round(floor, 5)
            r["expert_floor_frac"] = round(floor / fc1_ms, 4)
        return r
    fb = fc1_bytes(cfg, n_touched, rows)
    achieved = fb / (fc1_ms * 1e-3) / 1e9
    if cfg.experts == "mx":
        # 32-row expert tiles: activation rows staged in LDS once per 4-wavefront workgroup
        kern = ("mx_fc1_lds_kernel" if cfg.tile_m % 32 == 0 else "stream_gemm_mx_kernel") + \
            ", MXFP8 x MXFP4 scaled MFMA, SituGLU + MXFP8 requantization epilogue"
    else:
        kern = "stream_gemm_kernel, SituGLU epilogue"
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


def percentiles(xs):
    """Median, p10 and p90 (nearest rank) of a list of step times."""
    s = sorted(xs)
    n = len(s)

    def q(p):
        return s[min(n - 1, max(0, int(round(p * (n - 1)))))]
    return {"median": q(0.5), "p10": q(0.1), "p90": q(0.9)}


def graph_us_per_call(torch, call, reps=100, warm=10):
    """GPU time per call of `call` (library launches on the current stream): `reps` calls
    captured in a HIP graph, replayed once between two events; the host's launch rate
    does not enter."""
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            call()
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    best = None
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1000.0 / reps
        best = us if best is None else min(best, us)
    del graph
    return best


def route_microbench(torch, B, LI):
    """lmoe_route at T=1024, E=896, K=16 (us per call, algorithmic bytes), plus the grouped
    (8 groups, 4 kept) and Renormalize methods on the same logits."""
    cfg = LI.ROUTE_MASKED
    logits = LI.make_route_logits(cfg, 3, device="cuda")
    bias = LI.make_bias(cfg, 3, device="cuda")
    ids = torch.empty(cfg.T, cfg.K, dtype=torch.int32, device="cuda")
    w = torch.empty(cfg.T, cfg.K, dtype=torch.float32, device="cuda")
    calls = {
        "sigmoid": lambda: B.lmoe_route(cfg.T, cfg.E, cfg.K, logits, bias, cfg.rsf, 1, ids, w),
        "grouped_8_4": lambda: B.lmoe_route_grouped(cfg.T, cfg.E, cfg.K, 8, 4, logits, bias, cfg.rsf, 1, ids, w),
        "renormalize": lambda: B.lmoe_route_renormalize(cfg.T, cfg.E, cfg.K, logits, ids, w),
    }
    us = {name: graph_us_per_call(torch, call, reps=200) for name, call in calls.items()}
    nbytes = cfg.T * cfg.E * 4 + cfg.E * 4 + cfg.T * cfg.K * 8
    return us, nbytes, logits, bias


def permute_microbench(torch, B, ids, E, tile_m):
    """lmoe_permute on the given ids (device [T, K] int32): us per call."""
    T, K = ids.shape
    rc = B.lmoe_permute_rows_cap(T, E, K, tile_m)
    wsb = B.lmoe_permute_workspace_bytes(T, E, K)
    i32 = dict(dtype=torch.int32, device="cuda")
    o = [torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(E + 1, **i32), torch.empty(rc, **i32),
         torch.empty(rc // tile_m, **i32), torch.empty(T * K, **i32)]
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    return graph_us_per_call(torch, lambda: B.lmoe_permute(T, E, K, tile_m, ids, *o[:5], o[5], rc, ws, wsb),
                             reps=100), o[0]


def masked_situ_microbench(torch, B, LI, counts):
    """lmoe_situ_masked over the [E, T_max, 2d] bf16 buffer with per-expert valid counts
    v_e = min(count_e, T_max) from the routing histogram: us per call and algorithmic
    bytes (valid rows read, 2d bf16 each, and written, d bf16 each)."""
    cfg = LI.ROUTE_MASKED
    v = counts.clamp(0, cfg.T_max).to(torch.int32)
    x = LI.make_masked_input(cfg, 3, v.cpu(), device="cuda")
    out = torch.empty(cfg.E, cfg.T_max, cfg.d, dtype=torch.bfloat16, device="cuda")
    us = graph_us_per_call(torch, lambda: B.lmoe_situ_masked(cfg.E, cfg.T_max, cfg.d, B.LMOE_BF16, x, v,
                                                             cfg.beta, cfg.linear_beta, out), reps=100)
    nbytes = int(v.sum()) * (2 * cfg.d * 2 + cfg.d * 2) + cfg.E * 4
    return us, nbytes, int(v.sum())


def copy_bandwidth(torch, nbytes=FLUSH_BYTES):
    """Measured device copy bandwidth (read + write bytes per second) of a plain copy of
    `nbytes`, best of five."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, dst
    return 2 * nbytes / (best * 1e-3) / 1e9


def gpu_clock():
    """The GPU's shader (gfx) clock in MHz as amd-smi reports it right after the timed
    region (current, min and max of the first gfx clock domain), or the tool's error. Not
    under rocprofv3: the tool is a Python script started through `env`, and a child that
    inherits the profiler's preloaded library would replace itself after that library has
    opened the GPU."""
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        return {"skipped": "running under rocprofv3"}
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True, text=True,
                           timeout=20)
        if r.returncode != 0:
            return {"error": (r.stderr or r.stdout).strip()[:200]}
        found = {}

        def walk(o, path):
            if isinstance(o, dict):
                for k, v in o.items():
                    kl = str(k).lower()
                    if "gfx" in kl and isinstance(v, dict) and not found:
                        for kk in ("clk", "min_clk", "max_clk"):
                            vv = v.get(kk)
                            found[kk + "_mhz"] = vv.get("value") if isinstance(vv, dict) else vv
                        found["domain"] = str(k)
                    walk(v, path + [k])
            elif isinstance(o, list):
                for v in o:
                    walk(v, path)
        walk(json.loads(r.stdout), [])
        return found or {"raw": r.stdout.strip()[:400]}
    except Exception as e:  # noqa: BLE001 - reported, not fatal
        return {"error": str(e)[:200]}


def host_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count()}


def time_layer(torch, layer, Xs, steps, flush=None):
    """Per-step GPU times (ms) of `steps` layer steps, from events on the main stream
    around each step; inputs rotate over Xs. With `flush` (a device buffer), every step is
    preceded by a write of the whole buffer, outside the events."""
    stream = torch.cuda.current_stream()
    evs = []
    for i in range(steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        layer.forward(Xs[i % len(Xs)])
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def launch_modes(torch, layer, X, steps=200):
    """Microseconds per step, back to back, of the same layer step launched four ways: the
    Python sequence of library calls (the default), the library's own step
    (lmoe_layer_forward), the library's HIP graph of it (lmoe_layer_capture / _replay) and
    torch's HIP graph of the Python sequence."""
    import time

    def per_step(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return round((time.perf_counter() - t0) / steps * 1e6, 2)

    T = X.shape[0]
    nat = layer.native(T)
    cap = torch.cuda.Stream()              # stream capture needs a stream other than the default
    nat.capture(X, cap)
    g = layer.capture(X)
    res = {"python_eager": per_step(lambda: layer.forward(X)), "library_eager": per_step(lambda: nat.forward(X)),
           "library_graph": per_step(nat.replay), "torch_graph": per_step(g.replay)}
    torch.cuda.synchronize()
    nat.close()
    del g
    return res


_SPIN = {}


def spin_cycles_per_us(torch):
    """Clock cycles of torch.cuda._sleep (a one-wave kernel that spins on the clock and
    touches no memory) per microsecond, measured once with events."""
    if "c" not in _SPIN:
        n = 1 << 20
        torch.cuda._sleep(n)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(n)
        b.record()
        torch.cuda.synchronize()
        _SPIN["c"] = n / max(a.elapsed_time(b) * 1e3, 1.0)
    return _SPIN["c"]


def kernel_durations(torch, layer, Xs, steps, flush=None, spin_us=0):
    """Mean durations (ms) of each library call of the step (StepTimer events on the launch
    stream) over `steps` steps; with `flush`, a cache-clearing write precedes each step,
    with `spin_us` (and no flush) a spin of that many microseconds that touches no memory.
    Either keeps the GPU behind the host when the host's event bookkeeping takes longer
    than a step (decode): otherwise the GPU would wait for the host inside the first timed
    call of every step."""
    from latent_moe_layer_sigmoid_amd import StepTimer
    timer = StepTimer(torch.cuda.current_stream())
    spin = int(spin_cycles_per_us(torch) * spin_us) if flush is None and spin_us > 0 else 0
    for i in range(steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        elif spin:
            torch.cuda._sleep(spin)
        layer.forward(Xs[i % len(Xs)], timer=timer)
    torch.cuda.synchronize()
    return timer.durations()


def layer_record(torch, cfg, layer, Xs, steps, flush, seed):
    """Sub-record of one layer workload: per-step percentiles, tokens/s at the median,
    the layer's HBM fraction and the FC1 roofline (event-timed) for these steps."""
    for X in Xs:
        layer.forward(X)
    torch.cuda.synchronize()
    st = time_layer(torch, layer, Xs, steps, flush)
    pc = percentiles(st)
    # steps under 1 ms (decode) are shorter than the host's bookkeeping of the timed pass
    dur = kernel_durations(torch, layer, Xs, steps, flush, spin_us=500 if pc["median"] < 1.0 else 0)
    b = layer.buffers(cfg.T)
    counts = b["counts"].cpu()
    n_touched = int((counts > 0).sum())
    rows = int(b["tile_offsets"][-1].item())
    lb = layer_bytes(cfg, n_touched)
    roof = fc1_roofline(cfg, n_touched, rows, cfg.T * cfg.K, dur["fc1"])
    roof["traffic"] = fc1_traffic(cfg, seed) if len(Xs) == 1 and flush is None else None
    med = pc["median"]
    return {
        "tokens_per_s": round(cfg.T / (med * 1e-3), 1),
        "step_us": {k: round(v * 1e3, 2) for k, v in pc.items()},
        "layer_hbm": {"algorithmic_bytes": lb, "frac_at_median": round(lb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "kernels_us": {k: round(v * 1e3, 2) for k, v in dur.items()},
        "inputs": len(Xs),
        "steps": steps,
    }


def make_layer(torch, LI, cfg, seed, schedule, fold="auto"):
    from latent_moe_layer_sigmoid_amd import LatentMoELayer, LayerShape
    w = LI.make_layer_weights(cfg, seed, device="cuda")
    shape = LayerShape(H=cfg.H, L=cfg.L, E=cfg.E, K=cfg.K, d=cfg.d, I=cfg.I, dtype=cfg.dtype, experts=cfg.experts,
                       beta=cfg.beta, linear_beta=cfg.linear_beta, rsf=cfg.rsf, eps=cfg.eps, tile_m=cfg.tile_m)
    layer = LatentMoELayer(shape, w, shared_stream=schedule == "shared_stream",
                           router_stream=schedule == "router_stream",
                           fold_shared_fc2={"auto": None, "on": True, "off": False}[fold])
    del w
    torch.cuda.empty_cache()
    return layer


def cpu_baseline(torch, LI, cfg, seed, X_cpu, n_tokens, seconds=10.0):
    """The oracle timed on the host on `n_tokens` tokens of the same workload, its BLAS
    held to the host cores this process may run on."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import numpy as np

    import oracle
    from gpu_helpers import oracle_weights, run_oracle_layer
    cores = len(os.sched_getaffinity(0))
    w_cpu = LI.make_layer_weights(cfg, seed, device="cpu", experts=False)
    o = oracle_weights(cfg, seed, w_cpu)
    X64 = X_cpu[:n_tokens].to(torch.float64).numpy()
    with _blas_limit(cores):
        # expert weights are generated ahead of the timed region (the oracle reads arrays)
        ids, _, _ = oracle.route(oracle.router_logits(X64, o["W_r"]), o["bias"], cfg.K, cfg.rsf)
        for e in np.unique(ids):
            o["W1"][e], o["W2"][e]
        reps, t0 = 0, time.perf_counter()
        while True:      # repeat the sample until about `seconds` of CPU work
            run_oracle_layer(cfg, o, X64)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= seconds:
                break
    return reps * n_tokens / dt, dt, reps, cores


class _blas_limit:
    """Hold numpy's BLAS to n threads inside the block (threadpoolctl), when available."""

    def __init__(self, n):
        self.n, self.ctx = n, None

    def __enter__(self):
        try:
            from threadpoolctl import threadpool_limits
            self.ctx = threadpool_limits(limits=self.n, user_api="blas")
            self.ctx.__enter__()
        except Exception:  # noqa: BLE001
            self.ctx = None
        return self

    def __exit__(self, *a):
        if self.ctx is not None:
            self.ctx.__exit__(*a)


def oracle_route_us(LI, logits_cpu, bias_cpu, cores):
    """The oracle's routing (numpy float64) at T=1024, E=896, K=16: us per call with the
    BLAS held to one thread and to all cores (routing uses no BLAS product, so the two
    figures mainly show that)."""
    import oracle
    cfg = LI.ROUTE_MASKED
    lg = logits_cpu.double().numpy()
    b = bias_cpu.double().numpy()
    out = {}
    for name, n in (("1_core", 1), ("all_cores", cores)):
        with _blas_limit(n):
            oracle.route(lg, b, cfg.K, cfg.rsf)
            reps, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < 2.0:
                oracle.route(lg, b, cfg.K, cfg.rsf)
                reps += 1
            out[name] = round((time.perf_counter() - t0) * 1e6 / reps, 1)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_bf16", choices=["prefill_bf16", "decode_bf16", "mx_experts",
                                                                   "tiny_fp32"])
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the headline workload only (no sub-records of the other workloads)")
    ap.add_argument("--cpu-tokens", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB (fp32 multiply by one) before the "
                         "layer, as the reference kernel for HBM byte counters")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of the layer step instead of eager launches")
    ap.add_argument("--fold-shared-fc2", choices=["auto", "on", "off"], default="auto",
                    help="with a second stream: compute the shared FC2 inside the tail (on), on the side stream "
                         "(off), or by token count (auto: folded from 256 tokens)")
    ap.add_argument("--schedule", choices=["one_stream", "shared_stream", "router_stream"], default="shared_stream",
                    help="shared_stream: the shared expert runs on a second stream; router_stream: also the "
                         "router GEMM and routing on a third")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: this build has no multi-GPU "
              "path (the layer runs on one GPU's full share; see the sharding plan in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch

    import lmoe_inputs as LI
    from latent_moe_layer_sigmoid_amd import binding as B
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    B.lib()
    cfg = LI.CONFIGS[args.workload]
    log(f"workload {cfg.name}: generating weights on the GPU")
    layer = make_layer(torch, LI, cfg, args.seed, args.schedule, args.fold_shared_fc2)
    X_cpu = LI.make_x(cfg, args.seed)
    X = X_cpu.to("cuda")

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

    # per-step GPU times (events around each step) and per-call kernel durations (events on
    # the launch stream), in separate passes of the same number of steps
    st = percentiles(time_layer(torch, layer, [X], args.steps))
    dur = kernel_durations(torch, layer, [X], args.steps)

    b = layer.buffers(cfg.T)
    counts = b["counts"].cpu()
    n_touched = int((counts > 0).sum())
    rows = int(b["tile_offsets"][-1].item())
    fc1_ms = dur["fc1"]
    roof = fc1_roofline(cfg, n_touched, rows, cfg.T * cfg.K, fc1_ms, counts.tolist())
    roof["traffic"] = fc1_traffic(cfg, args.seed)
    lb = layer_bytes(cfg, n_touched)
    lf = layer_flops(cfg)
    log(f"n_touched={n_touched} rows={rows} fc1={fc1_ms * 1e3:.1f}us step={ms_per_step * 1e3:.1f}us "
        f"layer bytes={lb / 1e6:.1f}MB flops={lf / 1e9:.1f}G")
    log("per-step us: " + ", ".join(f"{k}={v * 1e3:.1f}" for k, v in dur.items()))
    clock = gpu_clock()

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
                               f"shared I={cfg.I} experts={cfg.experts} tile_m={cfg.tile_m}"
                               + (" skewed routing (hidden mean 0.5)" if cfg.x_mean else ""),
                   "tokens_per_step": cfg.T, "seed": args.seed, "schedule": args.schedule,
                   "launch": "hip_graph" if args.graph else "eager"},
        "roofline": roof,
        "step_us_events": {k: round(v * 1e3, 2) for k, v in st.items()},
        "layer_hbm": {"algorithmic_bytes": lb, "achieved_GBs": round(lb / (ms_per_step * 1e-3) / 1e9, 1),
                      "frac": round(lb / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "layer_mfma": {"algorithmic_flops": lf, "achieved_TFLOPs": round(lf / (ms_per_step * 1e-3) / 1e12, 1),
                       "frac": round(lf / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "kernels_us": {k: round(v * 1e3, 2) for k, v in dur.items()},
        "gpu_clock": clock,
    }

    if not args.no_extras:
        wl = {}
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        # decode: same packed weights, 16-row tiles, T=8 (the weights depend only on the seed)
        dec = LI.DECODE
        if cfg.experts == "dense" and cfg.dtype == "bf16" and cfg.H == dec.H:
            dl = layer.reshaped(tile_m=dec.tile_m)
            Xd = [LI.make_x(dec, args.seed + 100 * i).to("cuda") for i in range(4)]
            log("decode: warm (one input) and cold (1 GiB written before each step, 4 inputs)")
            wl["decode_bf16"] = {"config": f"T={dec.T} H={dec.H} L={dec.L} E={dec.E} top-{dec.K} d={dec.d} "
                                           f"shared I={dec.I} bf16 tile_m={dec.tile_m}",
                                 "warm": layer_record(torch, dec, dl, Xd[:1], 100, None, args.seed),
                                 "cold": layer_record(torch, dec, dl, Xd, 40, flush, args.seed),
                                 "launch_us_per_step": launch_modes(torch, dl, Xd[0])}
            del dl
        # prefill as a sub-record when the headline is another workload
        if cfg.name != "prefill_bf16" and cfg.experts == "dense" and cfg.dtype == "bf16":
            pf = LI.PREFILL
            pl = layer.reshaped(tile_m=pf.tile_m)
            Xp = [LI.make_x(pf, args.seed).to("cuda")]
            log("prefill sub-record")
            wl["prefill_bf16"] = {"warm": layer_record(torch, pf, pl, Xp, 10, None, args.seed)}
            del pl, Xp
        torch.cuda.synchronize()
        if cfg.name != "mx_experts":
            del layer
            torch.cuda.empty_cache()
            mx = LI.MX
            log("MX experts layer: generating weights")
            ml = make_layer(torch, LI, mx, args.seed, args.schedule)
            Xm = [LI.make_x(mx, args.seed + 100 * i).to("cuda") for i in range(4)]
            wl["mx_experts"] = {"config": f"T={mx.T} MXFP4 x MXFP8 experts, the rest bf16, tile_m={mx.tile_m}",
                                "warm": layer_record(torch, mx, ml, Xm[:1], 40, None, args.seed),
                                "cold": layer_record(torch, mx, ml, Xm, 20, flush, args.seed)}
            del ml, Xm
            torch.cuda.empty_cache()
        log("routing, permutation and masked SituGLU micro-benchmarks")
        route_all, route_bytes, rlogits, rbias = route_microbench(torch, B, LI)
        rc = LI.ROUTE_MASKED
        ids = torch.empty(rc.T, rc.K, dtype=torch.int32, device="cuda")
        wts = torch.empty(rc.T, rc.K, dtype=torch.float32, device="cuda")
        B.lmoe_route(rc.T, rc.E, rc.K, rlogits, rbias, rc.rsf, 1, ids, wts)
        perm_us, rcounts = permute_microbench(torch, B, ids, rc.E, 16)
        ms_us, ms_bytes, ms_rows = masked_situ_microbench(torch, B, LI, rcounts)
        pf_ids = b["ids"] if cfg.name == "prefill_bf16" else None
        wl["route_masked"] = {
            "config": f"T={rc.T} E={rc.E} top-{rc.K}; masked SituGLU [{rc.E}, {rc.T_max}, {2 * rc.d}] bf16",
            "route_us_per_call": {k: round(v, 3) for k, v in route_all.items()},
            "route_algorithmic_bytes": route_bytes,
            "route_hbm_frac": round(route_bytes / (route_all["sigmoid"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 5),
            "permute_us_per_call": {"T1024_tile16": round(perm_us, 3)},
            "masked_situglu": {"us_per_call": round(ms_us, 3), "valid_rows": ms_rows, "algorithmic_bytes": ms_bytes,
                               "hbm_frac": round(ms_bytes / (ms_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        }
        if pf_ids is not None:
            us, _ = permute_microbench(torch, B, pf_ids, cfg.E, cfg.tile_m)
            wl["route_masked"]["permute_us_per_call"]["T8192_tile128"] = round(us, 3)
        del flush
        torch.cuda.empty_cache()
        wl["copy_bandwidth_GBs"] = round(copy_bandwidth(torch), 1)
        res["workloads"] = wl
        res["route_us_per_call"] = wl["route_masked"]["route_us_per_call"]["sigmoid"]
        res["route_hbm_frac"] = wl["route_masked"]["route_hbm_frac"]
        res["host"] = host_info()

    if not args.no_cpu_baseline:
        n = min(args.cpu_tokens, cfg.T)
        log(f"cpu baseline: oracle on {n} tokens")
        v, dt, reps, cores = cpu_baseline(torch, LI, cfg, args.seed, X_cpu, n, args.cpu_seconds)
        cb = {"value": round(v, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
              "sample": f"{n} of the {cfg.T} tokens of one step ({n * cfg.K} expert pairs), repeated {reps}x, "
                        f"numpy float64 with BLAS held to {cores} threads, {dt:.1f} s"}
        if not args.no_extras:
            rc = LI.ROUTE_MASKED
            cb["route_us_per_call"] = oracle_route_us(LI, LI.make_route_logits(rc, 3), LI.make_bias(rc, 3), cores)
            cb["host"] = host_info()
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
