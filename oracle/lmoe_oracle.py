"""Plain, slow CPU oracle of the latent-MoE layer forward (numpy, float64).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the entry point's smoke check and
by the benchmark's CPU-baseline leg; never by the GPU product path, with which it
shares no code (its own number-format codecs, its own rounding, numpy/libm
transcendentals in float64).

Sources (page, then section):
  [P1] vLLM pull request 50088, "[MoE] Latent-MoE runner, fused MoE tail, SituGLU
       activation and single-group top-k routing", section "What's in it",
       commits 1 (single-group top-k), 2 (SituGLU), 3 (SituGLU through fused MoE),
       4 (DeepSeekV3 routing), 5 (SituGLU on dequantized values), 6 (fused tail),
       7 (LatentMoERunner).
  [P2] TensorRT-LLM pull request 20541 (Kimi K3 MoE decode, router stream),
       sections "Description" and "Commit 1: routing as its own op".
  [P3] vLLM API page vllm.models.kimi_k3.amd.latent_moe_runner, class
       ROCmLatentMoERunner: _fused_forward, _shard_up_proj_tail,
       enable_quantized_routed_input.
  [OCP-MX] OCP Microscaling Formats (MX) v1.0 specification (FP8 E4M3, FP4 E2M1,
       E8M0 scale, block size 32) -- the format behind the MXE4M3 x MXE2M1 runner
       that [P2] "Description" names.

Everything is computed in float64 from the exact input values. Values are rounded to
a storage dtype only where the GPU path stores a tensor across its C ABI: logits
(fp32), latent x, expert activation a, combined latent z (fp32), shared-expert output,
normalized latent n and the layer output. The FC1 pre-activation h is never rounded
(the fused kernel never stores it).

Parity pins: every function below is pinned in tests/test_oracle_pins.py against
closed forms, brute force, library routines on special cases or invariants.
"""
import numpy as np

# --------------------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------------------


def f32_round(x):
    """Round float64 values to the nearest float32 (IEEE round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_round(x):
    """Round float64 values directly to the nearest bfloat16 (8 significant bits,
    float32 exponent range), ties to even; values beyond the largest finite bf16
    become infinities."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, ex = np.frexp(xf)                       # |x| = m * 2**ex, m in [0.5, 1)
    q_exp = np.maximum(ex - 8, -133)           # 8-bit significand; subnormal quantum 2**-133
    q = np.ldexp(np.ones_like(xf), q_exp)
    y = np.rint(xf / q) * q                    # rint: round half to even
    y = np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, y), y)
    out[fin] = y
    return out


def round_to(x, dtype):
    """Round to a storage dtype: 'bf16', 'f32', or 'f64' (no rounding)."""
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f32":
        return f32_round(x)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


def bf16_bits_to_f64(bits):
    """Decode raw bfloat16 bit patterns (uint16) to float64."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e4m3_decode(codes):
    """[OCP-MX] FP8 E4M3 ("fn": no infinities, S.1111.111 is NaN): exponent bias 7,
    3 mantissa bits, exponent field 0 is subnormal (m * 2**-9)."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return s * mag


E4M3_MAX = 448.0


def e4m3_encode(v):
    """[OCP-MX] float64 -> FP8 E4M3 code: round to nearest, ties to even; magnitudes
    that round above 448 saturate to 448 (the MX conversion clamps). The sign bit is
    set for v < 0 (so a negative value that rounds to zero encodes as 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    E = ex - 1                                   # floor(log2 a) for a > 0
    quantum = np.ldexp(1.0, np.maximum(E, -6) - 3)
    q = np.rint(a / quantum) * quantum
    q = np.where(a > 0, q, 0.0)
    q = np.minimum(q, E4M3_MAX)
    # encode q (exactly representable now)
    _, qex = np.frexp(np.where(q > 0, q, 1.0))
    QE = qex - 1
    normal = q >= 2.0 ** -6
    mant_n = np.rint((q / np.ldexp(1.0, QE) - 1.0) * 8.0).astype(np.int64)
    code_n = ((QE + 7) << 3) | mant_n
    code_s = np.rint(q / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    code = np.where(v < 0, code | 0x80, code)
    return code.astype(np.uint8)


E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_decode(nibbles):
    """[OCP-MX] FP4 E2M1: sign bit 3, 2 exponent bits (bias 1), 1 mantissa bit;
    exponent field 0 is subnormal (m * 0.5)."""
    n = np.asarray(nibbles).astype(np.int64)
    s = np.where(n & 8, -1.0, 1.0)
    e = (n >> 1) & 3
    m = (n & 1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, e - 1))
    return s * mag


def e8m0_decode(b):
    """[OCP-MX] E8M0 scale: 2**(b - 127); 0xFF is NaN."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def mxfp4_dequant(codes, scales):
    """Packed MXFP4 -> float64. codes [..., n/2] (element 2i in the low nibble, 2i+1 in
    the high nibble), scales [..., n/32] e8m0, one per 32 consecutive elements."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes & 0xF
    hi = codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    vals = e2m1_decode(nib)
    sc = e8m0_decode(scales)
    n = vals.shape[-1]
    vals = vals.reshape(*vals.shape[:-1], n // 32, 32) * sc[..., None]
    return vals.reshape(*vals.shape[:-2], n)


def mxfp8_quantize(v):
    """[OCP-MX] quantization of float64 values [..., n] (n % 32 == 0) to MXFP8 E4M3.

    Per block of 32 consecutive elements: shared exponent
    X = floor(log2(max |v|)) - 8 (8 = largest E4M3 exponent), clamped to the E8M0
    range [-127, 127]; elements are v / 2**X rounded to E4M3 (ties to even,
    saturating at 448). An all-zero block gets X = 0 (scale byte 127)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    assert n % 32 == 0
    blk = v.reshape(*v.shape[:-1], n // 32, 32)
    amax = np.max(np.abs(blk), axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, ex - 1 - 8, 0)
    X = np.clip(X, -127, 127)
    codes = e4m3_encode(blk / np.ldexp(1.0, X)[..., None])
    return codes.reshape(v.shape), (X + 127).astype(np.uint8)


def mxfp8_dequant(codes, scales):
    """MXFP8 E4M3 codes [..., n] with e8m0 scales [..., n/32] -> float64."""
    vals = e4m3_decode(codes)
    n = vals.shape[-1]
    sc = e8m0_decode(scales)
    return (vals.reshape(*vals.shape[:-1], n // 32, 32) * sc[..., None]).reshape(vals.shape)


# --------------------------------------------------------------------------------------
# layer steps
# --------------------------------------------------------------------------------------


def linear(x, w):
    """x @ w^T in float64; weights are stored [out, in] (the nn.Linear layout that
    [P3] _shard_up_proj_tail multiplies by weight.t())."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def router_logits(X, W_r):
    """Router GEMM: fp32 logits [T, E] ([P2] "Description": the router GEMM runs
    first; [P1] commit 4: DeepSeekV3 routing takes FP32 logits)."""
    return f32_round(linear(X, W_r))


def route(logits, bias, K, rsf, renormalize=True):
    """Single-group DeepSeekV3 top-k routing ([P1] commits 1 and 4).

    With one group, the grouped rule reduces to the K best of every expert (commit 1).
    Scores are s = sigmoid(logits); experts are selected on the bias-corrected score
    kappa = s + bias, slot k holding the k-th largest (commit 1: result k sits in
    lane k), ties to the lower expert index. The selection key is formed in fp32,
    the precision of the routing kernel and of its fp32 logits (commit 4). Weights
    use the uncorrected scores of the selected experts, renormalized to sum to one,
    then scaled by the routed scaling factor (commit 4), computed in float64 and
    rounded to fp32.

    Returns ids int32 [T, K], weights (fp32 values) [T, K], kappa64 [T, E]."""
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    b = np.zeros(E) if bias is None else np.asarray(bias, dtype=np.float64)
    s = sigmoid(logits)
    kappa32 = f32_round(f32_round(s) + b[None, :])
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -kappa32), axis=-1)   # primary: kappa desc; then index asc
    ids = order[:, :K].astype(np.int32)
    sel = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    if renormalize:
        w = rsf * sel / np.sum(sel, axis=1, keepdims=True)
    else:
        w = rsf * sel
    return ids, f32_round(w), s + b[None, :]


def route_grouped(logits, bias, K, rsf, n_group, topk_group, renormalize=True):
    """Grouped DeepSeekV3 top-k routing, the general case that single-group routing
    specializes ([P1] commit 1: n_group == topk_group == 1 is the degenerate case of the
    grouped kernels; commit 4: sigmoid + grouped-topk with bias and group counts). The
    pages give no formula; the reading taken is DeepSeek-V3's published rule:

      kappa = fp32(fp32(sigmoid(logits)) + bias), experts cut into n_group contiguous
      groups of E / n_group; a group's score is the fp32 sum of its two largest kappa
      (its only kappa when groups hold one expert); the topk_group groups with the highest
      scores are kept (ties -> lower group index); ids are the K largest kappa among the
      kept groups' experts (ties -> lower expert index), in descending order; weights as
      in route() from the unbiased scores.

    Returns ids int32 [T, K], weights (fp32 values) [T, K], group scores [T, n_group]."""
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    assert E % n_group == 0 and 1 <= topk_group <= n_group
    gs = E // n_group
    assert K <= topk_group * gs
    b = np.zeros(E) if bias is None else np.asarray(bias, dtype=np.float64)
    s = sigmoid(logits)
    kappa32 = f32_round(f32_round(s) + b[None, :])
    grp = kappa32.reshape(T, n_group, gs)
    top = -np.sort(-grp, axis=2)
    gscore = f32_round(top[:, :, 0] + top[:, :, 1]) if gs > 1 else top[:, :, 0]
    gidx = np.broadcast_to(np.arange(n_group), (T, n_group))
    gorder = np.lexsort((gidx, -gscore), axis=-1)
    keep = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(keep, gorder[:, :topk_group], True, axis=1)
    cand = np.repeat(keep, gs, axis=1)
    masked = np.where(cand, kappa32, -np.inf)
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -masked), axis=-1)
    ids = order[:, :K].astype(np.int32)
    sel = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    w = rsf * sel / np.sum(sel, axis=1, keepdims=True) if renormalize else rsf * sel
    return ids, f32_round(w), gscore


def route_renormalize(logits, K):
    """The "Renormalize" routing method ([P1] commit 4: on that path the logits are cast
    to BF16 and no bias, group counts or routed scaling factor are used; [P2] "Test
    Coverage": Renormalize routing next to the DeepSeekV3 method). Reading taken: the
    K largest bf16 logits (ties -> lower expert index), in descending order, weighted by
    the softmax of the selected logits.

    Returns ids int32 [T, K], weights (fp32 values) [T, K]."""
    lb = bf16_round(np.asarray(logits, dtype=np.float64))
    T, E = lb.shape
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -lb), axis=-1)
    ids = order[:, :K].astype(np.int32)
    sel = np.take_along_axis(lb, ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    return ids, f32_round(ex / np.sum(ex, axis=1, keepdims=True))


def permute(ids, E, tile_m):
    """Expert-sorted permutation of the (token, slot) pairs (the per-expert row map
    the expert GEMMs and the combine consume, padded to a row tile; [P2] "Commit 1").

    Pair p = t*K + k. Pairs are stably sorted by expert id (token order inside each
    expert). Each expert's segment is padded to a multiple of tile_m rows.

    Returns dict: counts [E], offsets [E+1], tile_offsets [E+1], row_to_pair
    [tile_offsets[E]] (-1 on pad rows), pair_to_row [T*K]."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    padded = -(-counts // tile_m) * tile_m
    tile_offsets = np.concatenate([[0], np.cumsum(padded)])
    order = np.argsort(flat, kind="stable")
    e_sorted = flat[order]
    rank = np.arange(flat.size) - offsets[e_sorted]
    rows = tile_offsets[e_sorted] + rank
    row_to_pair = np.full(int(tile_offsets[E]), -1, dtype=np.int64)
    row_to_pair[rows] = order
    pair_to_row = np.empty(flat.size, dtype=np.int64)
    pair_to_row[order] = rows
    return dict(counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
                tile_offsets=tile_offsets.astype(np.int32),
                row_to_pair=row_to_pair.astype(np.int32),
                pair_to_row=pair_to_row.astype(np.int32))


def situglu(g, u, beta, linear_beta):
    """SituGLU ([P1] commit 2): gate_out = beta * tanh(g / beta) * sigmoid(g);
    up_out = linear_beta * tanh(u / linear_beta) if linear_beta > 0, else u
    ([P1] commit 3: linear_beta <= 0 means unset and passes up through);
    out = gate_out * up_out."""
    if not (beta > 0 and np.isfinite(beta)):
        raise ValueError("beta is required and must be a positive finite number")
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    gate = beta * np.tanh(g / beta) * sigmoid(g)
    up = linear_beta * np.tanh(u / linear_beta) if linear_beta > 0 else u
    return gate * up


def situ_glu_rows(h, beta, linear_beta):
    """SituGLU on [..., 2d] rows: gate = first d columns, up = last d ([P1] commit 2,
    dense [..., 2*d] layout; [P3] enable_quantized_routed_input excludes the
    interleaved gate/up layout)."""
    d = h.shape[-1] // 2
    return situglu(h[..., :d], h[..., d:], beta, linear_beta)


def situ_masked(inp, counts, beta, linear_beta, out, dtype="bf16"):
    """Masked SituGLU over the batched [E, T_max, 2d] layout ([P1] commit 2): for
    expert e only rows r < min(max(counts[e], 0), T_max) are computed; every other
    row of `out` is left exactly as it was. Returns the new out array."""
    inp = np.asarray(inp, dtype=np.float64)
    res = np.array(out, dtype=np.float64, copy=True)
    E, T_max, _ = inp.shape
    for e in range(E):
        v = int(min(max(int(counts[e]), 0), T_max))
        if v:
            res[e, :v] = round_to(situ_glu_rows(inp[e, :v], beta, linear_beta), dtype)
    return res


def rmsnorm(z, gamma, eps):
    """Latent RMSNorm on the full expert sum ([P1] commit 7: reduce before the
    output transform, which contains an RMSNorm; [P3] _shard_up_proj_tail applies
    transform.norm to the reduced latent): n = z / sqrt(mean(z**2) + eps) * gamma."""
    z = np.asarray(z, dtype=np.float64)
    ms = np.mean(z * z, axis=-1, keepdims=True)
    g = 1.0 if gamma is None else np.asarray(gamma, dtype=np.float64)
    return z / np.sqrt(ms + eps) * g


def tail(z, gamma, eps, W_up, shared, dtype):
    """RMSNorm then up projection with the shared-expert output added in the
    projection's epilogue ([P3] _shard_up_proj_tail: shared += latent @ W_up^T;
    [P1] commit 6: the up projection folds in the shared-expert add)."""
    n = round_to(rmsnorm(z, gamma, eps), dtype)
    up = linear(n, W_up)
    out = up if shared is None else np.asarray(shared, np.float64) + up
    return n, round_to(out, dtype)


def _expert_fc1(e, x_rows, W1, W1_scales, mx):
    w = mxfp4_dequant(W1[e], W1_scales[e]) if mx else np.asarray(W1[e], np.float64)
    return linear(x_rows, w)


def _expert_fc2(e, a_rows, W2, W2_scales, mx):
    w = mxfp4_dequant(W2[e], W2_scales[e]) if mx else np.asarray(W2[e], np.float64)
    return linear(a_rows, w)


def shared_expert(X, W_s1, W_s2, beta, linear_beta, dtype):
    """Always-on shared expert on the original hidden input ([P2] "Commit 2": the
    shared experts run beside the routed path; [P3] _fused_forward: the shared
    experts get the untransformed hidden states): SituGLU MLP, output rounded."""
    hs = linear(X, W_s1)
    a_s = round_to(situ_glu_rows(hs, beta, linear_beta), dtype)
    return round_to(linear(a_s, W_s2), dtype)


def layer_forward(X, W_r, bias, W_down, W1, W2, W_s1, W_s2, gamma, W_up, *,
                  K, rsf, beta, linear_beta, eps, dtype, mx=False,
                  W1_scales=None, W2_scales=None, renormalize=True,
                  routing="sigmoid", n_group=1, topk_group=1):
    """One latent-MoE layer forward for the token rows in X ([P2] "Description" step
    order: router GEMM, latent down projection, input quantization, routing, FC1 /
    FC2, then the routed reduction with RMSNorm and the latent up projection; [P1]
    commit 7 and [P3] _fused_forward / _shard_up_proj_tail for the latent tail).

    X: float64 [T, H] exact input values. W1[e] / W2[e]: per-expert weights, float64
    [2d, L] / [L, d], or (mx=True) packed MXFP4 codes with W1_scales[e] / W2_scales[e].
    Every token's output depends only on its own row, so a subset of tokens can be
    passed on its own. routing / n_group / topk_group select route_renormalize or
    route_grouped instead of single-group routing.

    Returns a dict of every intermediate the GPU path stores."""
    X = np.asarray(X, dtype=np.float64)
    T = X.shape[0]
    logits = router_logits(X, W_r)                                   # router GEMM
    if routing == "renormalize":                                     # routing
        ids, w = route_renormalize(logits, K)
        kappa = None
    elif n_group > 1:
        ids, w, _ = route_grouped(logits, bias, K, rsf, n_group, topk_group, renormalize)
        kappa = None
    else:
        ids, w, kappa = route(logits, bias, K, rsf, renormalize)
    x = round_to(linear(X, W_down), dtype)                           # latent down projection
    res = dict(logits=logits, ids=ids, weights=w, kappa=kappa, x=x)
    if mx:                                                           # input quantization
        xq, xs = mxfp8_quantize(x)
        x_in = mxfp8_dequant(xq, xs)
        res.update(xq=xq, xs=xs)
    else:
        x_in = x
    L = x.shape[1]
    Y = np.zeros((T, K, L))
    d = None
    act = None
    for e in np.unique(ids):                                         # routed experts
        tt, kk = np.nonzero(ids == e)
        h = _expert_fc1(int(e), x_in[tt], W1, W1_scales, mx)         # FC1 (never rounded)
        a = situ_glu_rows(h, beta, linear_beta)                      # SituGLU
        if d is None:
            d = a.shape[1]
            act = np.zeros((T, K, d))
            actq = np.zeros((T, K, d), dtype=np.uint8) if mx else None
            acts = np.zeros((T, K, d // 32), dtype=np.uint8) if mx else None
        if mx:                                                       # requantization
            aq, as_ = mxfp8_quantize(f32_round(a))
            a_in = mxfp8_dequant(aq, as_)
            actq[tt, kk] = aq
            acts[tt, kk] = as_
            act[tt, kk] = f32_round(a)
        else:
            a_in = round_to(a, dtype)
            act[tt, kk] = a_in
        Y[tt, kk] = _expert_fc2(int(e), a_in, W2, W2_scales, mx)     # FC2 (expert output)
    z = np.zeros((T, L))
    for k in range(K):                                               # weighted combine
        z = z + w[:, k:k + 1] * Y[:, k, :]
    z = f32_round(z)
    sh = shared_expert(X, W_s1, W_s2, beta, linear_beta, dtype)      # shared expert
    n, out = tail(z, gamma, eps, W_up, sh, dtype)                    # RMSNorm, up projection
    res.update(act=act, z=z, sh=sh, n=n, out=out)
    if mx:
        res.update(actq=actq, acts=acts)
    return res


def grouped_gaps_ok(kappa, gscore, K, n_group, topk_group, min_gap=1e-4):
    """Per token: True when the group decision and the expert decision are both clear:
    adjacent gaps among the topk_group + 1 largest group scores, and among the K + 1
    largest keys of the kept groups' experts, are at least min_gap."""
    kappa = np.asarray(kappa, dtype=np.float64)
    gscore = np.asarray(gscore, dtype=np.float64)
    T, E = kappa.shape
    gs = E // n_group
    gtop = -np.sort(-gscore, axis=1)[:, :topk_group + 1]
    ok = np.all(gtop[:, :-1] - gtop[:, 1:] >= min_gap, axis=1) if topk_group < n_group else np.ones(T, bool)
    gidx = np.broadcast_to(np.arange(n_group), (T, n_group))
    gorder = np.lexsort((gidx, -gscore), axis=-1)
    keep = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(keep, gorder[:, :topk_group], True, axis=1)
    masked = np.where(np.repeat(keep, gs, axis=1), kappa, -np.inf)
    top = -np.sort(-masked, axis=1)[:, :K + 1]
    gaps = top[:, :-1] - top[:, 1:]
    return ok & np.all(np.where(np.isfinite(gaps), gaps, np.inf) >= min_gap, axis=1)


def kappa_gaps_ok(kappa, K, min_gap=1e-4):
    """Per token: True when every adjacent gap among the K+1 largest selection keys
    is at least min_gap (the input guard that keeps the top-K set and its slot order
    away from rounding-level near-ties)."""
    kappa = np.asarray(kappa, dtype=np.float64)
    top = -np.sort(-kappa, axis=1)[:, :K + 1]
    gaps = top[:, :-1] - top[:, 1:]
    return np.all(gaps >= min_gap, axis=1)
