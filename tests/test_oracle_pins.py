"""Pins of the CPU oracle to facts that do not come from the oracle itself: hand-derived
closed forms (tests/golden/), brute force on tiny inputs, library routines on special
cases (torch's bf16 / fp8 conversions, plain Python loops) and invariants."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from golden_io import frac, lines, value

RNG = np.random.default_rng(1234)


# ------------------------------------------------------------------------- number formats

def test_bf16_round_matches_torch_on_fp32_inputs():
    x = np.concatenate([RNG.standard_normal(20000) * 10.0 ** RNG.integers(-30, 30, 20000),
                        RNG.standard_normal(1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_is_a_single_rounding_from_float64():
    # 1 + 2^-8 + 2^-30 lies above the midpoint 1 + 2^-8: direct rounding gives 1 + 2^-7
    # (rounding through fp32 first would land on the midpoint and tie to 1.0).
    assert oracle.bf16_round(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7
    assert oracle.bf16_round(1 + 2 ** -8) == 1.0                  # tie -> even
    assert oracle.bf16_round(1 + 3 * 2 ** -8) == 1 + 2 ** -6      # tie -> even (mantissa 2)
    assert oracle.bf16_round(-(1 + 3 * 2 ** -8)) == -(1 + 2 ** -6)
    assert np.isinf(oracle.bf16_round(3.5e38))


def test_bf16_bits_decode():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F80], dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), ref)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_e4m3_encode_matches_torch_in_range():
    mags = np.abs(RNG.standard_normal(50000)) * 2.0 ** RNG.integers(-12, 9, 50000)
    v = (np.where(RNG.random(50000) < 0.5, -1, 1) * mags).astype(np.float32)
    v = v[np.abs(v) <= 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(v.astype(np.float64))
    # torch keeps the sign of values that round to zero as well
    assert np.array_equal(got, ref)


def test_e4m3_golden_points():
    n = 0
    for ln in lines("mx_formats.txt"):
        f = ln.split()
        if f[0] == "e4m3":
            assert int(oracle.e4m3_encode(float(f[1]))) == int(f[2], 16), ln
            n += 1
    assert n >= 10


def test_e2m1_golden_table():
    n = 0
    for ln in lines("mx_formats.txt"):
        f = ln.split()
        if f[0] == "e2m1":
            assert oracle.e2m1_decode(int(f[1])) == float(f[2]), ln
            n += 1
    assert n == 10
    assert tuple(oracle.e2m1_decode(np.arange(8))) == oracle.E2M1_VALUES


def test_e8m0_decode():
    got = oracle.e8m0_decode(np.array([127, 0, 254, 120, 255]))
    assert got[0] == 1.0 and got[1] == 2.0 ** -127 and got[2] == 2.0 ** 127 and got[3] == 2.0 ** -7
    assert np.isnan(got[4])


def test_mxfp4_dequant_nibble_order_and_scale():
    codes = np.zeros((1, 16), dtype=np.uint8)
    codes[0, 0] = 0x21      # element 0: code 1 (0.5), element 1: code 2 (1.0)
    codes[0, 15] = 0xF7     # element 30: code 7 (6.0), element 31: code 15 (-6.0)
    got = oracle.mxfp4_dequant(codes, np.array([[128]], dtype=np.uint8))
    assert got[0, 0] == 1.0 and got[0, 1] == 2.0 and got[0, 30] == 12.0 and got[0, 31] == -12.0
    assert np.count_nonzero(got) == 4


def _mx_block(kind):
    b = np.zeros(32)
    if kind == "ones":
        b[:] = 1.0
    elif kind == "max448":
        b[5] = 448.0
    elif kind == "max480":
        b[:] = 1.0
        b[7] = 480.0
    elif kind == "max3":
        b[:] = 0.75
        b[3] = 3.0
    return b


def test_mxfp8_golden_blocks():
    n = 0
    for ln in lines("mx_formats.txt"):
        f = ln.split()
        if f[0] != "mxblock":
            continue
        b = _mx_block(f[1])
        codes, scales = oracle.mxfp8_quantize(b[None, :])
        imax = int(np.argmax(np.abs(b)))
        other = (imax + 1) % 32
        assert int(scales[0, 0]) == int(f[2]), ln
        assert int(codes[0, imax]) == int(f[3], 16), ln
        assert int(codes[0, other]) == int(f[4], 16), ln
        n += 1
    assert n == 5


def test_mxfp8_round_trip_of_representable_blocks():
    # codes whose block maximum has the top exponent field (values in [256, 448]) are
    # reproduced exactly by quantize(dequantize(.)): the shared exponent is recovered.
    rows = 200
    codes = RNG.integers(0, 256, size=(rows, 64)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10
    for r in range(rows):
        for b in range(2):
            codes[r, b * 32 + RNG.integers(0, 32)] = 0x78 | RNG.integers(0, 7) | (0x80 * RNG.integers(0, 2))
            blk = codes[r, b * 32:(b + 1) * 32]
            blk[(blk & 0x78) == 0x78] = blk[(blk & 0x78) == 0x78] & 0xFE  # top-binade codes below 0x7F
    scales = RNG.integers(100, 150, size=(rows, 2)).astype(np.uint8)
    v = oracle.mxfp8_dequant(codes, scales)
    c2, s2 = oracle.mxfp8_quantize(v)
    assert np.array_equal(s2, scales)
    # -0.0 and +0.0 both decode to 0; the encoder writes 0x00 for them
    canon = np.where((codes & 0x7F) == 0, 0, codes)
    assert np.array_equal(c2, canon)


def test_mxfp8_error_bound():
    v = RNG.standard_normal((64, 128)) * 10.0 ** RNG.integers(-3, 3, (64, 1))
    codes, scales = oracle.mxfp8_quantize(v)
    back = oracle.mxfp8_dequant(codes, scales)
    X = oracle.e8m0_decode(scales).repeat(32, axis=1)
    a = np.abs(v) / X
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    half_q = 0.5 * np.ldexp(1.0, np.maximum(ex - 1, -6) - 3) * X
    sat = a > 464.0
    assert np.all((np.abs(back - v) <= half_q) | sat)
    assert np.all(np.abs(back[sat]) == 448.0 * X[sat])


# ------------------------------------------------------------------------------- SituGLU

def test_situglu_golden_closed_forms():
    n = 0
    for ln in lines("situglu_closed_form.txt"):
        f = ln.split()
        g = float(frac(f[0])) * math.log(float(frac(f[1])))
        u = float(frac(f[2])) * math.log(float(frac(f[3])))
        beta, lb = float(frac(f[4])), float(frac(f[5]))
        out = oracle.situglu(g, u, beta, lb)
        gate = oracle.situglu(g, 1.0, beta, 0.0)
        up = oracle.situglu(math.log(3.0), u, 1.0, lb) / 0.6  # gate(ln3, beta=1) = 3/5 exactly
        assert gate == pytest.approx(value(f[6]), rel=1e-13, abs=1e-15), ln
        assert up == pytest.approx(value(f[7]), rel=1e-13, abs=1e-15), ln
        assert out == pytest.approx(value(f[8]), rel=1e-13, abs=1e-15), ln
        n += 1
    assert n >= 10


def test_situglu_odd_even_identities():
    g = RNG.standard_normal(1000) * 4
    for beta in (0.25, 1.0, 3.0):
        fp = oracle.situglu(g, 1.0, beta, 0.0)
        fm = oracle.situglu(-g, 1.0, beta, 0.0)
        t = beta * np.tanh(g / beta)
        np.testing.assert_allclose(fp - fm, t, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(fp + fm, t * np.tanh(g / 2.0), rtol=1e-10, atol=1e-14)


def test_situglu_large_beta_is_silu():
    g = np.linspace(-8, 8, 101)
    got = oracle.situglu(g, 1.0, 1e8, 0.0)
    silu = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    np.testing.assert_allclose(got, silu, rtol=1e-9, atol=1e-12)


def test_situglu_linear_beta_unset_passes_up_through():
    g = RNG.standard_normal(100)
    u = RNG.standard_normal(100) * 5
    base = oracle.situglu(g, 1.0, 1.5, 0.0)
    assert np.array_equal(oracle.situglu(g, u, 1.5, 0.0), base * u)
    assert np.array_equal(oracle.situglu(g, u, 1.5, -2.0), base * u)


def test_situglu_bounds_and_beta_required():
    g = RNG.standard_normal(1000) * 50
    u = RNG.standard_normal(1000) * 50
    out = oracle.situglu(g, u, 2.0, 0.5)
    assert np.all(np.abs(out) <= 2.0 * 0.5)
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            oracle.situglu(g, u, bad, 0.5)


def test_situglu_rows_gate_is_first_half():
    h = RNG.standard_normal((3, 8))
    got = oracle.situ_glu_rows(h, 1.0, 0.5)
    assert np.array_equal(got, oracle.situglu(h[:, :4], h[:, 4:], 1.0, 0.5))
    assert not np.allclose(got, oracle.situglu(h[:, 4:], h[:, :4], 1.0, 0.5))


def test_situ_masked_leaves_pad_rows_untouched():
    E, Tm, d = 5, 6, 8
    inp = RNG.standard_normal((E, Tm, 2 * d))
    out0 = np.full((E, Tm, d), np.nan)
    out0[0, 0, 0] = 123.0
    counts = np.array([0, 3, 6, 9, -2])
    res = oracle.situ_masked(inp, counts, 1.0, 0.5, out0)
    for e, c in enumerate(counts):
        v = min(max(c, 0), Tm)
        np.testing.assert_array_equal(res[e, v:], out0[e, v:])
        assert np.array_equal(res[e, :v], oracle.bf16_round(oracle.situ_glu_rows(inp[e, :v], 1.0, 0.5)))


# ------------------------------------------------------------------------------- routing

def _rational_logits(tok):
    return [math.log(float(frac(t))) for t in tok]


def test_route_golden_rational_example():
    K = rsf = None
    bias, logits, ids, ws = None, {}, {}, {}
    for ln in lines("routing_rational.txt"):
        f = ln.split()
        if f[0] == "K":
            K = int(f[1])
        elif f[0] == "rsf":
            rsf = float(f[1])
        elif f[0] == "bias":
            bias = np.array([float(x) for x in f[1:]], dtype=np.float32).astype(np.float64)
        elif f[0] == "logit":
            logits[int(f[1])] = _rational_logits(f[2:])
        elif f[0] == "ids":
            ids[int(f[1])] = [int(x) for x in f[2:]]
        elif f[0] == "w":
            ws[int(f[1])] = [float(frac(x)) for x in f[2:]]
    L = oracle.f32_round(np.array([logits[t] for t in sorted(logits)]))
    got_ids, got_w, _ = oracle.route(L, bias, K, rsf)
    for t in sorted(logits):
        assert list(got_ids[t]) == ids[t]
        np.testing.assert_allclose(got_w[t], ws[t], rtol=1e-6)
    # the weights are NOT the bias-corrected scores
    assert not np.allclose(got_w[0], [0.95 * 2 / 2.625, 0.875 * 2 / 2.625, 0.8 * 2 / 2.625], rtol=1e-3)


def _brute_force_topk(kappa_row, K):
    """The unique ordered K-subset whose members beat every non-member on
    (key desc, index asc), found by enumerating all subsets."""
    E = len(kappa_row)
    beats = lambda i, j: kappa_row[i] > kappa_row[j] or (kappa_row[i] == kappa_row[j] and i < j)
    found = []
    for sub in itertools.combinations(range(E), K):
        rest = [j for j in range(E) if j not in sub]
        if all(beats(i, j) for i in sub for j in rest):
            found.append(sub)
    assert len(found) == 1
    order = list(found[0])
    # selection sort on the same relation
    res = []
    while order:
        best = order[0]
        for i in order[1:]:
            if beats(i, best):
                best = i
        res.append(best)
        order.remove(best)
    return res


def _read_routing_golden(name):
    d = dict(logits={}, ids={}, w={}, gscore={})
    for ln in lines(name):
        f = ln.split()
        if f[0] in ("K", "n_group", "topk_group"):
            d[f[0]] = int(f[1])
        elif f[0] == "rsf":
            d["rsf"] = float(f[1])
        elif f[0] == "bias":
            d["bias"] = np.array([float(x) for x in f[1:]], dtype=np.float32).astype(np.float64)
        elif f[0] == "logit":
            d["logits"][int(f[1])] = f[2:]
        elif f[0] == "ids":
            d["ids"][int(f[1])] = [int(x) for x in f[2:]]
        elif f[0] in ("w", "gscore"):
            d[f[0]][int(f[1])] = [float(frac(x)) if "/" in x or x.isdigit() else float(x) for x in f[2:]]
    return d


def test_route_grouped_golden_rational_example():
    d = _read_routing_golden("grouped_routing.txt")
    L = oracle.f32_round(np.array([_rational_logits(d["logits"][t]) for t in sorted(d["logits"])]))
    ids, w, gscore = oracle.route_grouped(L, d["bias"], d["K"], d["rsf"], d["n_group"], d["topk_group"])
    for t in sorted(d["logits"]):
        assert list(ids[t]) == d["ids"][t]
        np.testing.assert_allclose(w[t], d["w"][t], rtol=1e-6)
        np.testing.assert_allclose(gscore[t], d["gscore"][t], rtol=1e-6)
    # the group stage matters here: plain top-3 picks differently
    plain, _, _ = oracle.route(L, d["bias"], d["K"], d["rsf"])
    assert list(plain[0]) != d["ids"][0] and list(plain[1]) != d["ids"][1]


def test_route_grouped_reduces_to_single_group():
    rng = np.random.default_rng(21)
    lg = rng.standard_normal((40, 64)) * 1.4
    b = rng.uniform(-0.05, 0.05, 64)
    ids, w, _ = oracle.route(lg, b, 8, 2.5)
    for n_group in (1, 4, 8):   # one group, or every group kept
        gi, gw, _ = oracle.route_grouped(lg, b, 8, 2.5, n_group, n_group)
        assert np.array_equal(gi, ids) and np.array_equal(gw, w)


@pytest.mark.parametrize("trial", range(20))
def test_route_grouped_matches_brute_force(trial):
    """Group choice and expert choice by enumeration of all subsets (tiny E)."""
    rng = np.random.default_rng(300 + trial)
    n_group, gs = int(rng.integers(2, 5)), int(rng.integers(1, 4))
    E = n_group * gs
    topk_group = int(rng.integers(1, n_group + 1))
    K = int(rng.integers(1, topk_group * gs + 1))
    lg = oracle.f32_round(rng.standard_normal((1, E)) * 2)
    b = np.array(rng.uniform(-0.1, 0.1, E), dtype=np.float32).astype(np.float64)
    ids, _, gscore = oracle.route_grouped(lg, b, K, 1.0, n_group, topk_group)
    kap = oracle.f32_round(oracle.f32_round(oracle.sigmoid(lg[0])) + b)
    # group scores: the two largest members, by pairwise enumeration
    for g in range(n_group):
        mem = kap[g * gs:(g + 1) * gs]
        best = max(mem) if gs == 1 else max(oracle.f32_round(mem[i] + mem[j])
                                             for i, j in itertools.combinations(range(gs), 2))
        assert gscore[0, g] == best
    kept = _brute_force_topk(gscore[0], topk_group)
    cand = [e for e in range(E) if e // gs in kept]
    sub = _brute_force_topk(kap[cand], K)
    assert list(ids[0]) == [cand[i] for i in sub]


def test_route_renormalize_golden():
    d = _read_routing_golden("renormalize_routing.txt")
    L = np.array([[float(x) for x in d["logits"][t]] for t in sorted(d["logits"])])
    ids, w = oracle.route_renormalize(L, d["K"])
    for t in sorted(d["logits"]):
        assert list(ids[t]) == d["ids"][t]
        np.testing.assert_allclose(w[t], d["w"][t], rtol=1e-7)


def test_route_renormalize_invariants():
    rng = np.random.default_rng(5)
    lg = oracle.f32_round(rng.standard_normal((50, 96)) * 2)
    ids, w = oracle.route_renormalize(lg, 6)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-6)
    lb = oracle.bf16_round(lg)
    # ids: the top-6 of the bf16 logits by a stable sort; weights: the full softmax renormalized
    assert np.array_equal(ids, np.argsort(-lb, axis=1, kind="stable")[:, :6])
    full = np.exp(lb - lb.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-6)
    i1, w1 = oracle.route_renormalize(lg, 1)
    assert np.all(w1 == 1.0) and np.array_equal(i1[:, 0], np.argmax(lb, axis=1))


@pytest.mark.parametrize("trial", range(60))
def test_route_matches_brute_force_with_ties(trial):
    rng = np.random.default_rng(trial)
    E = int(rng.integers(2, 10))
    K = int(rng.integers(1, min(4, E) + 1))
    T = 3
    if trial % 3 == 0:   # integer logits and biases: many exact ties
        logits = rng.integers(-2, 3, (T, E)).astype(np.float64)
        bias = rng.integers(-1, 2, E).astype(np.float64) * 0.25
    else:
        logits = oracle.f32_round(rng.standard_normal((T, E)) * 2)
        bias = oracle.f32_round(rng.uniform(-0.05, 0.05, E))
    ids, w, _ = oracle.route(logits, bias, K, 2.5)
    kappa32 = oracle.f32_round(oracle.f32_round(1.0 / (1.0 + np.exp(-logits))) + bias)
    for t in range(T):
        assert list(ids[t]) == _brute_force_topk(list(kappa32[t]), K)
    np.testing.assert_allclose(w.sum(1), 2.5, rtol=1e-6)


def test_route_equal_keys_pick_lower_index():
    logits = np.zeros((2, 8))
    ids, _, _ = oracle.route(logits, np.zeros(8), 3, 1.0)
    assert ids.tolist() == [[0, 1, 2], [0, 1, 2]]
    bias = np.array([0, 0.5, 0, 0.5, 0, 0, 0.5, 0])
    ids, _, _ = oracle.route(logits, bias, 4, 1.0)
    assert ids[0].tolist() == [1, 3, 6, 0]


def test_route_special_cases():
    rng = np.random.default_rng(7)
    logits = oracle.f32_round(rng.standard_normal((16, 12)) * 2)
    bias = oracle.f32_round(rng.uniform(-0.05, 0.05, 12))
    s = 1.0 / (1.0 + np.exp(-logits))
    # K = 1: the weight is the scaling factor itself
    _, w1, _ = oracle.route(logits, bias, 1, 2.5)
    assert np.all(w1 == np.float32(2.5))
    # K = E: every expert, weights rsf * s / sum(s)
    ids, wE, _ = oracle.route(logits, bias, 12, 1.0)
    assert all(sorted(r) == list(range(12)) for r in ids.tolist())
    np.testing.assert_allclose(np.take_along_axis(wE, np.argsort(ids, 1), 1),
                               s / s.sum(1, keepdims=True), rtol=1e-6)
    # no bias: top-K of the logits themselves (sigmoid is monotone)
    ids0, _, _ = oracle.route(logits, None, 4, 1.0)
    for t in range(16):
        assert list(ids0[t]) == [int(i) for i in np.argsort(-logits[t], kind="stable")[:4]]
    # without renormalization the weight is rsf * s
    idsn, wn, _ = oracle.route(logits, bias, 4, 2.0, renormalize=False)
    np.testing.assert_allclose(wn, 2.0 * np.take_along_axis(s, idsn.astype(int), 1), rtol=1e-6)


def test_route_expert_relabeling():
    rng = np.random.default_rng(11)
    logits = oracle.f32_round(rng.standard_normal((10, 20)) * 2)
    bias = oracle.f32_round(rng.uniform(-0.05, 0.05, 20))
    perm = rng.permutation(20)
    ids, w, _ = oracle.route(logits, bias, 5, 1.0)
    ids_p, w_p, _ = oracle.route(logits[:, perm], bias[perm], 5, 1.0)
    assert np.array_equal(perm[ids_p], ids)
    assert np.array_equal(w_p, w)


def test_kappa_gap_guard():
    kappa = np.array([[0.9, 0.8, 0.79995, 0.1], [0.9, 0.8, 0.7, 0.1]])
    assert oracle.kappa_gaps_ok(kappa, 2).tolist() == [False, True]
    assert oracle.kappa_gaps_ok(kappa, 1).tolist() == [True, True]


# --------------------------------------------------------------------------- permutation

def _loop_permute(ids, E, tile_m):
    T, K = ids.shape
    rows, tile_off, counts = [], [0], []
    for e in range(E):
        seg = [t * K + k for t in range(T) for k in range(K) if ids[t, k] == e]
        counts.append(len(seg))
        pad = (-len(seg)) % tile_m
        rows += seg + [-1] * pad
        tile_off.append(len(rows))
    return counts, tile_off, rows


@pytest.mark.parametrize("T,E,K,tile_m", [(1, 4, 2, 1), (7, 5, 3, 4), (33, 16, 4, 16),
                                          (64, 64, 8, 16), (5, 3, 3, 8), (0, 4, 2, 16)])
def test_permute_matches_loops(T, E, K, tile_m):
    rng = np.random.default_rng(T * 100 + E)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]) if T else np.zeros((0, K), int)
    p = oracle.permute(ids, E, tile_m)
    counts, tile_off, rows = _loop_permute(ids, E, tile_m)
    assert p["counts"].tolist() == counts
    assert p["tile_offsets"].tolist() == tile_off
    assert p["row_to_pair"].tolist() == rows
    assert p["offsets"].tolist() == [0] + list(np.cumsum(counts))
    assert p["counts"].sum() == T * K
    if T:
        back = p["row_to_pair"][p["pair_to_row"]]
        assert np.array_equal(back, np.arange(T * K))
        assert np.all(np.asarray(p["tile_offsets"]) % tile_m == 0)


# ----------------------------------------------------------------------- GEMMs and tail

def test_linear_matches_python_loops():
    x = RNG.standard_normal((3, 5))
    w = RNG.standard_normal((4, 5))
    got = oracle.linear(x, w)
    for i in range(3):
        for j in range(4):
            ref = 0.0
            for k in range(5):
                ref += x[i, k] * w[j, k]
            assert got[i, j] == pytest.approx(ref, rel=1e-14, abs=1e-14)
    assert np.array_equal(oracle.linear(x, np.eye(5)), x)


def test_rmsnorm_golden_closed_forms():
    n = 0
    for ln in lines("rmsnorm_closed_form.txt"):
        z, eps, gamma, exp = [p.split() for p in ln.split("|")]
        got = oracle.rmsnorm(np.array([float(v) for v in z])[None, :], np.array([float(v) for v in gamma]),
                             float(eps[0]))
        np.testing.assert_allclose(got[0], [float(frac(v)) for v in exp], rtol=1e-14, atol=1e-15)
        n += 1
    assert n == 4


def test_rmsnorm_invariants():
    z = RNG.standard_normal((5, 64)) * 3
    gamma = RNG.uniform(0.9, 1.1, 64)
    eps = 1e-2
    n = oracle.rmsnorm(z, gamma, eps)
    ms = np.mean(z * z, axis=1)
    np.testing.assert_allclose(np.mean((n / gamma) ** 2, axis=1), ms / (ms + eps), rtol=1e-12)
    np.testing.assert_allclose(oracle.rmsnorm(7 * z, gamma, 0.0), oracle.rmsnorm(z, gamma, 0.0), rtol=1e-12)
    assert np.all(oracle.rmsnorm(np.zeros((1, 8)), None, 1e-6) == 0)


def test_tail_shared_add_and_zero_projection():
    z = RNG.standard_normal((2, 16))
    sh = oracle.bf16_round(RNG.standard_normal((2, 8)))
    _, out = oracle.tail(z, None, 1e-6, np.zeros((8, 16)), sh, "bf16")
    assert np.array_equal(out, sh)
    W = RNG.standard_normal((8, 16))
    _, out_nosh = oracle.tail(z, None, 1e-6, W, None, "f64")
    _, out_sh = oracle.tail(z, None, 1e-6, W, sh, "f64")
    np.testing.assert_allclose(out_sh - out_nosh, sh, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------ full layer

def _closed_form_layer():
    ln3, ln7 = math.log(3.0), math.log(7.0)
    X = np.array([[ln3, 1, 0, 0], [-ln3, 1, 0, 0]], dtype=np.float64)
    W_r = np.array([[1, 0, 0, 0], [0, 0, 0, 0], [-1, 0, 0, 0], [0, ln7, 0, 0]], dtype=np.float64)
    bias = np.array([0, 0, 0.7, 0], dtype=np.float32).astype(np.float64)
    b = [[1, 1, 1, 1], [2, 2, 2, 2], [1, 2, 0, 0], [3, 0, 1, 0]]
    W1 = np.zeros((4, 8, 4))
    for e in range(4):
        W1[e, :4, 0] = 1.0
        for j in range(4):
            W1[e, 4 + j, 1] = b[e][j]
    W2 = np.stack([np.eye(4)] * 4)
    W_s1 = np.array([[1, 0, 0, 0], [1, 0, 0, 0], [0, 1, 0, 0], [0, 1, 0, 0]], dtype=np.float64)
    W_s2 = np.array([[1, 0], [0, 1], [0, 0], [1, 1]], dtype=np.float64)
    return dict(X=X, W_r=W_r, bias=bias, W_down=np.eye(4), W1=W1, W2=W2, W_s1=W_s1, W_s2=W_s2,
                gamma=np.ones(4), W_up=np.eye(4))


def test_layer_golden_closed_form():
    p = _closed_form_layer()
    res = oracle.layer_forward(p["X"], p["W_r"], p["bias"], p["W_down"], p["W1"], p["W2"], p["W_s1"],
                               p["W_s2"], p["gamma"], p["W_up"], K=2, rsf=2.0, beta=1.0,
                               linear_beta=0.0, eps=0.25, dtype="f64")
    rows = list(lines("layer_closed_form.txt"))
    assert len(rows) == 2
    for ln in rows:
        tok, ids, ws, z, out = [s.split() for s in ln.split("|")]
        t = int(tok[0])
        assert res["ids"][t].tolist() == [int(i) for i in ids]
        np.testing.assert_allclose(res["weights"][t], [value(v) for v in ws], rtol=1e-6)
        np.testing.assert_allclose(res["z"][t], [value(v) for v in z], rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(res["out"][t], [value(v) for v in out], rtol=1e-6, atol=1e-7)


def test_layer_normalizes_after_the_sum():
    # normalizing each expert's output before the weighted sum would give out - sh = rsf * sqrt(2)
    # on the first token's two nonzero channels (all experts identical here); summing first gives sqrt(2)
    p = _closed_form_layer()
    W1 = np.zeros((4, 8, 4))
    W1[:, :4, 0] = 1.0
    W1[:, 4, 1] = 1.0
    W1[:, 5, 1] = 1.0
    res = oracle.layer_forward(p["X"][:1], p["W_r"], p["bias"], p["W_down"], W1, p["W2"], p["W_s1"],
                               np.zeros((4, 2)), p["gamma"], p["W_up"], K=2, rsf=2.0, beta=1.0,
                               linear_beta=0.0, eps=0.0, dtype="f64")
    np.testing.assert_allclose(res["out"][0], [math.sqrt(2), math.sqrt(2), 0, 0], rtol=1e-12, atol=1e-14)


def _random_layer(T=6, H=32, L=16, E=8, K=3, d=8, I=8, seed=0, mx=False):
    rng = np.random.default_rng(seed)
    r = lambda *s: oracle.bf16_round(rng.standard_normal(s) / math.sqrt(s[-1]))
    p = dict(X=oracle.bf16_round(rng.standard_normal((T, H))), W_r=r(E, H) * 1.4,
             bias=oracle.f32_round(rng.uniform(-0.05, 0.05, E)), W_down=r(L, H),
             W_s1=r(2 * I, H), W_s2=r(H, I), gamma=oracle.bf16_round(rng.uniform(0.9, 1.1, L)),
             W_up=r(H, L))
    if mx:
        p["W1"] = rng.integers(0, 256, (E, 2 * d, L // 2)).astype(np.uint8)
        p["W1_scales"] = rng.integers(119, 123, (E, 2 * d, L // 32)).astype(np.uint8)
        p["W2"] = rng.integers(0, 256, (E, L, d // 2)).astype(np.uint8)
        p["W2_scales"] = rng.integers(119, 123, (E, L, d // 32)).astype(np.uint8)
    else:
        p["W1"] = r(E, 2 * d, L)
        p["W2"] = r(E, L, d)
    return p


def _run(p, X=None, mx=False):
    return oracle.layer_forward(p["X"] if X is None else X, p["W_r"], p["bias"], p["W_down"], p["W1"],
                                p["W2"], p["W_s1"], p["W_s2"], p["gamma"], p["W_up"], K=3, rsf=2.5,
                                beta=1.0, linear_beta=0.5 if not mx else 0.0, eps=1e-6, dtype="bf16",
                                mx=mx, W1_scales=p.get("W1_scales"), W2_scales=p.get("W2_scales"))


@pytest.mark.parametrize("mx", [False, True])
def test_layer_per_token_independence_and_order(mx):
    p = _random_layer(mx=mx, L=32, d=32)
    full = _run(p, mx=mx)
    sub = _run(p, X=p["X"][[4, 1]], mx=mx)
    assert np.array_equal(sub["out"], full["out"][[4, 1]])
    assert np.array_equal(sub["ids"], full["ids"][[4, 1]])
    perm = np.array([5, 3, 1, 0, 2, 4])
    pr = _run(p, X=p["X"][perm], mx=mx)
    assert np.array_equal(pr["out"], full["out"][perm])


def test_layer_routing_scale_only_through_eps():
    # RMSNorm(c * z) = RMSNorm(z) up to eps: the scaling factor is nearly invisible at the output
    p = _random_layer()
    a = _run(p)
    b = oracle.layer_forward(p["X"], p["W_r"], p["bias"], p["W_down"], p["W1"], p["W2"], p["W_s1"],
                             p["W_s2"], p["gamma"], p["W_up"], K=3, rsf=1.0, beta=1.0, linear_beta=0.5,
                             eps=1e-6, dtype="bf16")
    np.testing.assert_allclose(b["z"] * 2.5, a["z"], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(b["out"], a["out"], rtol=2e-2, atol=2e-2)


def test_layer_mx_uses_quantized_operands():
    p = _random_layer(mx=True, L=32, d=32)
    res = _run(p, mx=True)
    x_codes, x_scales = oracle.mxfp8_quantize(res["x"])
    assert np.array_equal(res["xq"], x_codes) and np.array_equal(res["xs"], x_scales)
    # FC1 of the first pair reproduced from the dequantized operands
    t, k = 0, 0
    e = int(res["ids"][t, k])
    W1 = oracle.mxfp4_dequant(p["W1"][e], p["W1_scales"][e])
    h = oracle.mxfp8_dequant(x_codes[t], x_scales[t]) @ W1.T
    a = oracle.f32_round(oracle.situ_glu_rows(h, 1.0, 0.0))
    np.testing.assert_array_equal(res["act"][t, k], a)
    aq, as_ = oracle.mxfp8_quantize(a[None, :])
    assert np.array_equal(res["actq"][t, k], aq[0]) and np.array_equal(res["acts"][t, k], as_[0])
