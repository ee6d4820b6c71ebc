"""Seeded synthetic workloads for the latent-MoE layer forward.

Shared by the GPU path (tests, benchmark) and by the CPU oracle's tests. It makes input
tensors only: none of the layer's arithmetic lives here.

Distributions (second argument of N is the variance): hidden X ~ N(x_mean, 1); the
router weight ~ N(0, logit_var / H) so that logits ~ N(0, logit_var); every other
weight ~ N(0, 1 / fan_in); selection bias ~ U(-b, b) in fp32; RMSNorm gamma
~ U(0.9, 1.1). MXFP4 expert weights are drawn directly in encoded form (codes from a
quantised-normal table, scale exponents spread over three adjacent powers of two).
"""
import math

import torch

from .configs import CONFIGS, CONFIG_ORDER, DECODE, MX, PREFILL, ROUTE_MASKED, TINY, LayerConfig, scaled
from .gen import (TID, mxfp4_codes, mxfp4_scales, normal, normal_rows, stream_key,
                  uniform)

__all__ = ["CONFIGS", "CONFIG_ORDER", "TINY", "DECODE", "ROUTE_MASKED", "PREFILL", "MX",
           "LayerConfig", "scaled", "torch_dtype", "weight_std", "make_x", "make_layer_weights",
           "expert_weight", "make_route_logits", "make_bias", "make_masked_input",
           "BF16_SENTINEL"]

BF16_SENTINEL = 0xFFC1   # a bf16 NaN pattern marking rows that must stay untouched


def torch_dtype(cfg: LayerConfig):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def weight_std(cfg: LayerConfig):
    return dict(
        W_r=math.sqrt(cfg.logit_var / cfg.H) if cfg.H else 0.0,
        W_down=1.0 / math.sqrt(cfg.H) if cfg.H else 0.0,
        W1=1.0 / math.sqrt(cfg.L) if cfg.L else 0.0,
        W2=1.0 / math.sqrt(cfg.d),
        W_s1=1.0 / math.sqrt(cfg.H) if cfg.H else 0.0,
        W_s2=1.0 / math.sqrt(cfg.I) if cfg.I else 0.0,
        W_up=1.0 / math.sqrt(cfg.L) if cfg.L else 0.0,
    )


def make_x(cfg: LayerConfig, seed: int, attempts=None, device="cpu", rows=None):
    """Hidden input rows [T, H]; row t is drawn from attempt attempts[t]."""
    rows = torch.arange(cfg.T) if rows is None else torch.as_tensor(rows)
    if attempts is None:
        attempts = torch.zeros(cfg.T, dtype=torch.int64)
    att = torch.as_tensor(attempts)[rows]
    return normal_rows(seed, TID["X"], rows, cfg.H, att, std=1.0, mean=cfg.x_mean,
                       dtype=torch_dtype(cfg), device=device)


def make_bias(cfg: LayerConfig, seed: int, device="cpu"):
    return uniform(seed, TID["bias"], cfg.E, -cfg.bias_range, cfg.bias_range).to(device)


def make_route_logits(cfg: LayerConfig, seed: int, attempts=None, device="cpu"):
    """fp32 router logits [T, E] ~ N(0, logit_var), drawn directly (routing microbench)."""
    if attempts is None:
        attempts = torch.zeros(cfg.T, dtype=torch.int64)
    return normal_rows(seed, TID["logits"], torch.arange(cfg.T), cfg.E, torch.as_tensor(attempts),
                       std=math.sqrt(cfg.logit_var), dtype=torch.float32, device=device)


def _dense(seed, name, shape, std, dtype, device):
    n = 1
    for s in shape:
        n *= s
    return normal(seed, TID[name], n, std, dtype=dtype, device=device).view(*shape)


def make_layer_weights(cfg: LayerConfig, seed: int, device="cpu", experts=True):
    """Every layer weight. experts=False skips W1 / W2 (the large per-expert tensors)."""
    dt = torch_dtype(cfg)
    sd = weight_std(cfg)
    w = dict(
        W_r=_dense(seed, "W_r", (cfg.E, cfg.H), sd["W_r"], dt, device),
        bias=make_bias(cfg, seed, device),
        W_down=_dense(seed, "W_down", (cfg.L, cfg.H), sd["W_down"], dt, device),
        W_s1=_dense(seed, "W_s1", (2 * cfg.I, cfg.H), sd["W_s1"], dt, device),
        W_s2=_dense(seed, "W_s2", (cfg.H, cfg.I), sd["W_s2"], dt, device),
        gamma=uniform(seed, TID["gamma"], cfg.L, 0.9, 1.1, dtype=dt).to(device),
        W_up=_dense(seed, "W_up", (cfg.H, cfg.L), sd["W_up"], dt, device),
    )
    if experts:
        if cfg.experts == "mx":
            for name, (n_out, n_in) in (("W1", (2 * cfg.d, cfg.L)), ("W2", (cfg.L, cfg.d))):
                nb = cfg.E * n_out * n_in
                w[name + "_codes"] = mxfp4_codes(seed, TID[name + "_codes"], nb // 2, sd[name],
                                                 device=device).view(cfg.E, n_out, n_in // 2)
                w[name + "_scales"] = mxfp4_scales(seed, TID[name + "_scales"], nb // 32, sd[name],
                                                   device=device).view(cfg.E, n_out, n_in // 32)
        else:
            w["W1"] = _dense(seed, "W1", (cfg.E, 2 * cfg.d, cfg.L), sd["W1"], dt, device)
            w["W2"] = _dense(seed, "W2", (cfg.E, cfg.L, cfg.d), sd["W2"], dt, device)
    return w


def expert_weight(cfg: LayerConfig, seed: int, name: str, e: int, device="cpu"):
    """One expert's slice of W1 ([2d, L]) or W2 ([L, d]); for MX configs a pair
    (codes [n_out, n_in/2], scales [n_out, n_in/32]). Bit-identical to the slice of the
    full tensor."""
    sd = weight_std(cfg)
    n_out, n_in = (2 * cfg.d, cfg.L) if name == "W1" else (cfg.L, cfg.d)
    per = n_out * n_in
    if cfg.experts == "mx":
        c = mxfp4_codes(seed, TID[name + "_codes"], per // 2, sd[name], device=device,
                        start=e * (per // 2)).view(n_out, n_in // 2)
        s = mxfp4_scales(seed, TID[name + "_scales"], per // 32, sd[name], device=device,
                         start=e * (per // 32)).view(n_out, n_in // 32)
        return c, s
    return normal(seed, TID[name], per, sd[name], dtype=torch_dtype(cfg), device=device,
                  start=e * per).view(n_out, n_in)


def make_masked_input(cfg: LayerConfig, seed: int, counts, device="cpu"):
    """Batched [E, T_max, 2d] bf16 activation buffer: rows r < min(counts[e], T_max) ~ N(0,1),
    every other row filled with the NaN sentinel."""
    E, Tm, n = cfg.E, cfg.T_max, 2 * cfg.d
    x = normal(seed, TID["masked_in"], E * Tm * n, 1.0, dtype=torch.bfloat16,
               device=device).view(E, Tm, n)
    v = torch.as_tensor(counts).clamp(0, Tm).to(device)
    pad = torch.arange(Tm, device=device)[None, :] >= v[:, None]
    xi = x.view(torch.int16)
    xi[pad] = torch.tensor(BF16_SENTINEL - 65536, dtype=torch.int16, device=device)
    return x
