"""Shared helpers of the parity tests: seeded inputs (with the oracle's top-k gap guard),
lazy per-expert weight banks for the oracle, and error metrics.

Inputs come from lmoe_inputs; expected values only from the oracle."""
import numpy as np
import torch

import lmoe_inputs as LI
import oracle

MIN_GAP = 1e-4


def f64(t):
    """Exact float64 copy of a tensor (bf16 and fp32 widen exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def norm_err(gpu, ref):
    """max |gpu - ref| / max |ref| (the layer-output tolerance metric)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / (den if den > 0 else 1.0))


def bf16_ulp_diff(a_bits, b_bits):
    """Max distance in bf16 units in the last place between two bf16 bit arrays."""
    def ordered(x):
        x = np.asarray(x).astype(np.int64) & 0xFFFF
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return int(np.max(np.abs(ordered(a_bits) - ordered(b_bits)))) if np.size(a_bits) else 0


class ExpertBank:
    """Per-expert weight slices generated on the CPU on first use (float64 for dense
    experts, packed codes or scale bytes for MX), so the oracle touches only the experts
    the sampled tokens route to."""

    def __init__(self, cfg, seed, name, part=None):
        self.cfg, self.seed, self.name, self.part = cfg, seed, name, part
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            w = LI.expert_weight(self.cfg, self.seed, self.name, e)
            if self.cfg.experts == "mx":
                w = w[0] if self.part == "codes" else w[1]
                self.cache[e] = w.numpy()
            else:
                self.cache[e] = w.to(torch.float64).numpy()
        return self.cache[e]


def guarded_route_logits(cfg, seed, max_rounds=100):
    """fp32 logits [T, E] (cpu) whose oracle selection keys have every adjacent gap among
    each token's top K+1 >= MIN_GAP; failing rows are redrawn with the next attempt."""
    bias = LI.make_bias(cfg, seed)
    b64 = bias.double().numpy()
    att = torch.zeros(cfg.T, dtype=torch.int64)
    logits = LI.make_route_logits(cfg, seed, att)
    for _ in range(max_rounds):
        _, _, kappa = oracle.route(logits.double().numpy(), b64, cfg.K, cfg.rsf)
        bad = ~oracle.kappa_gaps_ok(kappa, cfg.K, MIN_GAP)
        if not bad.any():
            return logits, bias, att
        att[torch.from_numpy(bad)] += 1
        logits = LI.make_route_logits(cfg, seed, att)
    raise RuntimeError("gap guard did not converge")


def guarded_x(cfg, seed, W_r64, b64, max_rounds=40):
    """Hidden rows X [T, H] (cpu) passing the oracle's top-k gap guard; rows whose
    routing keys have a near-tie are redrawn with attempt + 1."""
    att = torch.zeros(cfg.T, dtype=torch.int64)
    X = LI.make_x(cfg, seed, att)
    rows = np.arange(cfg.T)
    for _ in range(max_rounds):
        lg = oracle.router_logits(f64(X[torch.from_numpy(rows)]), W_r64)
        if cfg.routing == "renormalize":   # decisions on exactly cast bf16 values: no guard
            ok = np.ones(len(rows), dtype=bool)
        elif cfg.n_group > 1:
            _, _, gsc = oracle.route_grouped(lg, b64, cfg.K, cfg.rsf, cfg.n_group, cfg.topk_group)
            kappa = oracle.f32_round(oracle.f32_round(oracle.sigmoid(lg)) + b64[None, :])
            ok = oracle.grouped_gaps_ok(kappa, gsc, cfg.K, cfg.n_group, cfg.topk_group, MIN_GAP)
        else:
            _, _, kappa = oracle.route(lg, b64, cfg.K, cfg.rsf)
            ok = oracle.kappa_gaps_ok(kappa, cfg.K, MIN_GAP)
        rows = rows[~ok]
        if rows.size == 0:
            return X, att
        att[torch.from_numpy(rows)] += 1
        X[torch.from_numpy(rows)] = LI.make_x(cfg, seed, att, rows=torch.from_numpy(rows))
    raise RuntimeError("gap guard did not converge")


def oracle_weights(cfg, seed, w_cpu):
    """Oracle views of the layer weights: float64 dense arrays plus lazy expert banks."""
    o = {k: f64(v) for k, v in w_cpu.items() if k not in ("W1", "W2") and not k.startswith(("W1_", "W2_"))}
    if cfg.experts == "mx":
        o["W1"] = ExpertBank(cfg, seed, "W1", "codes")
        o["W1_scales"] = ExpertBank(cfg, seed, "W1", "scales")
        o["W2"] = ExpertBank(cfg, seed, "W2", "codes")
        o["W2_scales"] = ExpertBank(cfg, seed, "W2", "scales")
    else:
        o["W1"] = ExpertBank(cfg, seed, "W1")
        o["W2"] = ExpertBank(cfg, seed, "W2")
    return o


def oracle_route(cfg, logits64, b64):
    """The oracle's routing (ids, weights) for the config's routing method."""
    if cfg.routing == "renormalize":
        return oracle.route_renormalize(logits64, cfg.K)
    if cfg.n_group > 1:
        ids, w, _ = oracle.route_grouped(logits64, b64, cfg.K, cfg.rsf, cfg.n_group, cfg.topk_group)
        return ids, w
    ids, w, _ = oracle.route(logits64, b64, cfg.K, cfg.rsf)
    return ids, w


def run_oracle_layer(cfg, o, X64):
    return oracle.layer_forward(X64, o["W_r"], o["bias"], o["W_down"], o["W1"], o["W2"], o["W_s1"], o["W_s2"],
                                o["gamma"], o["W_up"], K=cfg.K, rsf=cfg.rsf, beta=cfg.beta,
                                linear_beta=cfg.linear_beta, eps=cfg.eps, dtype=cfg.dtype,
                                mx=cfg.experts == "mx", W1_scales=o.get("W1_scales"),
                                W2_scales=o.get("W2_scales"), routing=cfg.routing, n_group=cfg.n_group,
                                topk_group=cfg.topk_group)


def tile_expert_from_offsets(tile_offsets, tile_m, n_tiles):
    """Expected tile -> expert map from the oracle's tile offsets."""
    te = np.full(n_tiles, -1, dtype=np.int64)
    for e in range(len(tile_offsets) - 1):
        te[tile_offsets[e] // tile_m: tile_offsets[e + 1] // tile_m] = e
    return te
