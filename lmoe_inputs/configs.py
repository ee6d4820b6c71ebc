"""The five latent-MoE workloads: shapes, dtypes and layer hyper-parameters.

Symbols: T tokens, H hidden, L latent, E routed experts, K experts per token, d
expert intermediate size, I shared-expert intermediate size, beta / linear_beta the
SituGLU parameters (vLLM PR 50088, "SituGLU (situ_and_mul)", commit 2), rsf the
routed scaling factor (same PR, commit 4: DeepSeekV3 routing arguments).
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    L: int
    E: int
    K: int
    d: int
    I: int
    dtype: str            # "f32" or "bf16": activations and dense weights
    experts: str          # "dense" (same dtype as above) or "mx" (MXFP4 weights, MXFP8 activations)
    beta: float
    linear_beta: float    # <= 0 means unset: the up half passes through
    rsf: float
    bias_range: float     # selection bias ~ U(-bias_range, bias_range)
    logit_var: float      # router logits ~ N(0, logit_var) (second argument read as variance)
    x_mean: float = 0.0   # hidden ~ N(x_mean, 1); 0.5 skews the expert histogram
    eps: float = 1e-6
    tile_m: int = 16
    routing: str = "sigmoid"   # "sigmoid" (bias-corrected, DeepSeekV3) or "renormalize" (bf16 logits, softmax)
    n_group: int = 1      # grouped top-k (sigmoid routing): expert groups and groups kept
    topk_group: int = 1
    kind: str = "layer"   # "layer" or "route_masked"
    T_max: int = 0        # masked-activation buffer depth (route_masked only)
    notes: str = field(default="", compare=False)


TINY = LayerConfig(
    name="tiny_fp32", T=4, H=256, L=128, E=16, K=4, d=64, I=128, dtype="f32",
    experts="dense", beta=1.0, linear_beta=0.0, rsf=1.0, bias_range=0.1,
    logit_var=1.0, notes="fp32 weights and activations; parity scale")

DECODE = LayerConfig(
    name="decode_bf16", T=8, H=7168, L=2048, E=896, K=16, d=512, I=4096, dtype="bf16",
    experts="dense", beta=1.0, linear_beta=0.5, rsf=2.5, bias_range=0.05,
    logit_var=2.0, notes="HBM-bound on touched-expert weight reads")

ROUTE_MASKED = LayerConfig(
    name="route_masked", T=1024, H=0, L=0, E=896, K=16, d=512, I=0, dtype="bf16",
    experts="dense", beta=1.0, linear_beta=0.5, rsf=2.5, bias_range=0.05,
    logit_var=2.0, kind="route_masked", T_max=64,
    notes="fp32 logits given directly; masked SituGLU over [E, T_max, 2d] bf16")

PREFILL = LayerConfig(
    name="prefill_bf16", T=8192, H=7168, L=2048, E=896, K=16, d=512, I=4096, dtype="bf16",
    experts="dense", beta=1.0, linear_beta=0.5, rsf=2.5, bias_range=0.05,
    logit_var=2.0, x_mean=0.5, tile_m=128,
    notes="skewed token-to-expert load via a constant mean on the hidden input")

MX = LayerConfig(
    name="mx_experts", T=1024, H=7168, L=2048, E=896, K=16, d=512, I=4096, dtype="bf16",
    experts="mx", beta=1.0, linear_beta=0.0, rsf=2.5, bias_range=0.05,
    logit_var=2.0, tile_m=32,
    notes="expert weights MXFP4 (e2m1 + e8m0 per 32 along K); activations MXFP8 e4m3")

CONFIGS = {c.name: c for c in (TINY, DECODE, ROUTE_MASKED, PREFILL, MX)}
CONFIG_ORDER = [TINY, DECODE, ROUTE_MASKED, PREFILL, MX]


def scaled(cfg: LayerConfig, **over) -> LayerConfig:
    """A copy of `cfg` with some fields replaced (used for reduced parity shapes)."""
    d = dict(cfg.__dict__)
    d.update(over)
    return LayerConfig(**d)
