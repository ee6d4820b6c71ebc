"""Parity of each HIP kernel (through the C ABI) against the CPU oracle on the same
seeded inputs: bit-exact for ids, permutation, counts and MX codes; toleranced for
floating point."""
import math

import numpy as np
import pytest
import torch

import lmoe_inputs as LI
import oracle
from gpu_helpers import bf16_ulp_diff, f64, guarded_route_logits, norm_err, tile_expert_from_offsets

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def B():
    from latent_moe_layer_sigmoid_amd import binding
    binding.lib()
    return binding


# ----------------------------------------------------------------------------- routing

def _run_route(B, logits, bias, K, rsf, renorm=1):
    T, E = logits.shape
    ids = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, K), float("nan"), dtype=torch.float32, device=DEV)
    B.lmoe_route(T, E, K, logits.to(DEV), None if bias is None else bias.to(DEV), rsf, renorm, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("E,K,T", [(16, 4, 4), (16, 16, 9), (64, 8, 33), (100, 6, 50), (256, 16, 70),
                                   (300, 64, 17), (512, 1, 40), (896, 16, 1024), (1000, 32, 65), (1024, 64, 8)])
def test_route_matches_oracle(B, E, K, T):
    cfg = LI.scaled(LI.ROUTE_MASKED, T=T, E=E, K=K)
    if K == 64:   # 64 guarded gaps per token: a narrower logit spread keeps the guard satisfiable
        cfg = LI.scaled(cfg, logit_var=0.25)
    logits, bias, _ = guarded_route_logits(cfg, seed=1000 + E + K, max_rounds=400)
    ids, w = _run_route(B, logits, bias, K, cfg.rsf)
    rid, rw, _ = oracle.route(logits.double().numpy(), bias.double().numpy(), K, cfg.rsf)
    assert np.array_equal(ids, rid)
    np.testing.assert_allclose(w, rw, rtol=1e-5, atol=0)


def test_route_full_microbench_shape_both_seeds(B):
    for seed in (3, 103):
        cfg = LI.ROUTE_MASKED
        logits, bias, att = guarded_route_logits(cfg, seed)
        ids, w = _run_route(B, logits, bias, cfg.K, cfg.rsf)
        rid, rw, _ = oracle.route(logits.double().numpy(), bias.double().numpy(), cfg.K, cfg.rsf)
        assert np.array_equal(ids, rid)
        np.testing.assert_allclose(w, rw, rtol=1e-5)
        np.testing.assert_allclose(w.sum(1), cfg.rsf, rtol=1e-5)


def test_route_ties_pick_lower_index(B):
    T, E, K = 6, 896, 16
    logits = torch.zeros(T, E)
    bias = torch.zeros(E)
    bias[[5, 700, 64, 3]] = 0.25            # four raised experts, then ties among the rest
    logits[1, 800:] = 1.0                   # token 1: a tied block at the top
    logits[2, ::7] = -1.0
    ids, w = _run_route(B, logits, bias, K, 2.5)
    rid, rw, _ = oracle.route(logits.double().numpy(), bias.double().numpy(), K, 2.5)
    assert np.array_equal(ids, rid)
    assert ids[0].tolist() == [3, 5, 64, 700, 0, 1, 2, 4, 6, 7, 8, 9, 10, 11, 12, 13]
    np.testing.assert_allclose(w, rw, rtol=1e-5)


def test_route_no_bias_no_renormalize_and_k_equals_e(B):
    cfg = LI.scaled(LI.ROUTE_MASKED, T=40, E=64, K=64)
    logits, _, _ = guarded_route_logits(LI.scaled(cfg, K=63), seed=77)
    ids, w = _run_route(B, logits, None, 64, 1.5, renorm=0)
    rid, rw, _ = oracle.route(logits.double().numpy(), None, 64, 1.5, renormalize=False)
    assert np.array_equal(ids, rid)
    np.testing.assert_allclose(w, rw, rtol=1e-5)


def test_route_deterministic_and_empty(B):
    cfg = LI.scaled(LI.ROUTE_MASKED, T=256)
    logits, bias, _ = guarded_route_logits(cfg, seed=5)
    a = _run_route(B, logits, bias, cfg.K, cfg.rsf)
    b = _run_route(B, logits, bias, cfg.K, cfg.rsf)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    B.lmoe_route(0, 896, 16, None, None, 1.0, 1, None, None)    # T == 0: no-op



@pytest.mark.parametrize("T,E,K", [(4, 16, 4), (50, 256, 8), (1024, 896, 16), (9, 1000, 64), (33, 64, 64)])
def test_route_renormalize_matches_oracle(B, T, E, K):
    """Renormalize routing: ids bit-exact (decisions on exactly cast bf16 logits, ties to
    the lower index on both sides), softmax weights within 1e-5."""
    cfg = LI.scaled(LI.ROUTE_MASKED, T=T, E=E, K=K)
    logits = LI.make_route_logits(cfg, 4000 + E + K)
    ids = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, K), float("nan"), device=DEV)
    B.lmoe_route_renormalize(T, E, K, logits.to(DEV), ids, w)
    torch.cuda.synchronize()
    rid, rw = oracle.route_renormalize(logits.double().numpy(), K)
    assert np.array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-5, atol=0)


def _guarded_grouped_logits(cfg, seed, n_group, topk_group, max_rounds=200):
    bias = LI.make_bias(cfg, seed)
    att = torch.zeros(cfg.T, dtype=torch.int64)
    for _ in range(max_rounds):
        logits = LI.make_route_logits(cfg, seed, att)
        lg = logits.double().numpy()
        _, _, gsc = oracle.route_grouped(lg, bias.double().numpy(), cfg.K, cfg.rsf, n_group, topk_group)
        kap = oracle.f32_round(oracle.f32_round(oracle.sigmoid(lg)) + bias.double().numpy()[None, :])
        bad = ~oracle.grouped_gaps_ok(kap, gsc, cfg.K, n_group, topk_group)
        if not bad.any():
            return logits, bias
        att[torch.from_numpy(bad)] += 1
    raise RuntimeError("gap guard did not converge")


@pytest.mark.parametrize("T,E,K,n_group,topk_group", [(64, 256, 8, 8, 4), (40, 896, 16, 8, 4), (33, 64, 6, 64, 8),
                                                      (20, 120, 16, 4, 2), (16, 1024, 64, 16, 8), (8, 256, 8, 8, 8),
                                                      (8, 896, 16, 1, 1)])
def test_route_grouped_matches_oracle(B, T, E, K, n_group, topk_group):
    cfg = LI.scaled(LI.ROUTE_MASKED, T=T, E=E, K=K)
    if K == 64:
        cfg = LI.scaled(cfg, logit_var=0.25)
    logits, bias = _guarded_grouped_logits(cfg, 5000 + E + K, n_group, topk_group)
    ids = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, K), float("nan"), device=DEV)
    B.lmoe_route_grouped(T, E, K, n_group, topk_group, logits.to(DEV), bias.to(DEV), cfg.rsf, 1, ids, w)
    torch.cuda.synchronize()
    rid, rw, _ = oracle.route_grouped(logits.double().numpy(), bias.double().numpy(), K, cfg.rsf, n_group,
                                      topk_group)
    assert np.array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-5, atol=0)


def test_route_grouped_and_renormalize_checks(B):
    f = torch.zeros(64, device=DEV)
    z = torch.zeros(64, dtype=torch.int32, device=DEV)
    B.lmoe_route_grouped(0, 16, 4, 4, 2, None, None, 1.0, 1, None, None)       # T == 0: no-op
    B.lmoe_route_renormalize(0, 16, 4, None, None, None)
    for args, st in [((2, 16, 4, 3, 2), B.LMOE_ERR_INVALID_ARG),    # E % n_group != 0
                     ((2, 16, 9, 4, 2), B.LMOE_ERR_INVALID_ARG),    # K > topk_group * group size
                     ((2, 16, 4, 4, 5), B.LMOE_ERR_INVALID_ARG),    # topk_group > n_group
                     ((2, 2048, 4, 4, 2), B.LMOE_ERR_UNSUPPORTED)]:
        with pytest.raises(B.LmoeError) as ei:
            B.lmoe_route_grouped(*args, f, None, 1.0, 1, z, f)
        assert ei.value.status == st
    with pytest.raises(B.LmoeError) as ei:
        B.lmoe_route_renormalize(2, 4, 8, f, z, f)
    assert ei.value.status == B.LMOE_ERR_INVALID_ARG


# --------------------------------------------------------------------------- permutation

def _random_ids(T, E, K, rng, skew=0.0):
    if skew:
        p = np.exp(rng.standard_normal(E) * skew)
        p /= p.sum()
        ids = np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)])
    else:
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :K]
    return ids.astype(np.int32)


def _run_permute(B, ids, E, tile_m):
    T, K = ids.shape
    rc = B.lmoe_permute_rows_cap(T, E, K, tile_m)
    wsb = B.lmoe_permute_workspace_bytes(T, E, K)
    i32 = dict(dtype=torch.int32, device=DEV)
    o = dict(counts=torch.full((E,), -9, **i32), offsets=torch.full((E + 1,), -9, **i32),
             tile_offsets=torch.full((E + 1,), -9, **i32), row_to_pair=torch.full((rc,), -9, **i32),
             tile_expert=torch.full((rc // tile_m,), -9, **i32), pair_to_row=torch.full((T * K,), -9, **i32))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=DEV)
    B.lmoe_permute(T, E, K, tile_m, torch.from_numpy(ids).to(DEV), o["counts"], o["offsets"], o["tile_offsets"],
                   o["row_to_pair"], o["tile_expert"], o["pair_to_row"], rc, ws, wsb)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}, rc


@pytest.mark.parametrize("T,E,K,tile_m,skew", [(4, 16, 4, 16, 0), (8, 896, 16, 16, 0), (64, 896, 16, 16, 1.0),
                                               (65, 100, 16, 32, 0), (1024, 896, 16, 16, 0.7),
                                               (3000, 512, 8, 128, 1.5), (8192, 896, 16, 128, 1.0),
                                               (777, 1024, 64, 256, 0.3), (1, 1, 1, 16, 0),
                                               # padded row totals past 32767 while the row capacity
                                               # stays below 65536 (one packed 16 + 16-bit scan):
                                               # several blocks, and the single-block kernel
                                               (2048, 896, 16, 16, 0), (3000, 896, 16, 16, 0.3),
                                               (64, 896, 16, 64, 0)])
def test_permute_matches_oracle(B, T, E, K, tile_m, skew):
    rng = np.random.default_rng(T * 7 + E)
    ids = _random_ids(T, E, K, rng, skew)
    got, rc = _run_permute(B, ids, E, tile_m)
    ref = oracle.permute(ids, E, tile_m)
    nrows = int(ref["tile_offsets"][E])
    assert np.array_equal(got["counts"], ref["counts"])
    assert np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["tile_offsets"], ref["tile_offsets"])
    assert np.array_equal(got["row_to_pair"][:nrows], ref["row_to_pair"])
    assert np.array_equal(got["pair_to_row"], ref["pair_to_row"])
    assert np.array_equal(got["tile_expert"], tile_expert_from_offsets(ref["tile_offsets"], tile_m, rc // tile_m))
    # permute then unpermute is the identity
    assert np.array_equal(got["row_to_pair"][got["pair_to_row"]], np.arange(T * K))


@pytest.mark.parametrize("T,E,K,tile_m", [(4, 16, 4, 16), (8, 896, 16, 16), (16, 896, 16, 16), (17, 896, 16, 16),
                                           (1, 8, 8, 16), (8, 1024, 64, 32), (64, 256, 16, 128), (300, 896, 16, 128),
                                           (16, 896, 16, 128), (2048, 896, 16, 16)])
def test_route_permute_matches_oracle(B, T, E, K, tile_m):
    """One call = routing then permutation: fused into one workgroup for T <= 16 and
    T*K <= 1024, two kernels otherwise; both bit-exact against the oracle."""
    cfg = LI.scaled(LI.ROUTE_MASKED, T=T, E=E, K=K)
    if K == 64:
        cfg = LI.scaled(cfg, logit_var=0.25)
    logits, bias, _ = guarded_route_logits(cfg, seed=2000 + T + E + K, max_rounds=400)
    rc = B.lmoe_permute_rows_cap(T, E, K, tile_m)
    wsb = B.lmoe_permute_workspace_bytes(T, E, K)
    i32 = dict(dtype=torch.int32, device=DEV)
    ids = torch.full((T, K), -7, **i32)
    w = torch.full((T, K), float("nan"), dtype=torch.float32, device=DEV)
    o = dict(counts=torch.full((E,), -9, **i32), offsets=torch.full((E + 1,), -9, **i32),
             tile_offsets=torch.full((E + 1,), -9, **i32), row_to_pair=torch.full((rc,), -9, **i32),
             tile_expert=torch.full((rc // tile_m,), -9, **i32), pair_to_row=torch.full((T * K,), -9, **i32))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=DEV)
    B.lmoe_route_permute(T, E, K, logits.to(DEV), bias.to(DEV), cfg.rsf, 1, ids, w, tile_m, o["counts"], o["offsets"],
                         o["tile_offsets"], o["row_to_pair"], o["tile_expert"], o["pair_to_row"], rc, ws, wsb)
    torch.cuda.synchronize()
    rid, rw, _ = oracle.route(logits.double().numpy(), bias.double().numpy(), K, cfg.rsf)
    assert np.array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-5, atol=0)
    ref = oracle.permute(rid, E, tile_m)
    got = {k: v.cpu().numpy() for k, v in o.items()}
    nrows = int(ref["tile_offsets"][E])
    for k in ("counts", "offsets", "tile_offsets", "pair_to_row"):
        assert np.array_equal(got[k], ref[k]), k
    assert np.array_equal(got["row_to_pair"][:nrows], ref["row_to_pair"])
    assert np.array_equal(got["tile_expert"], tile_expert_from_offsets(ref["tile_offsets"], tile_m, rc // tile_m))


def test_route_permute_empty_and_checks(B):
    i32 = dict(dtype=torch.int32, device=DEV)
    z = torch.zeros(64, **i32)
    f = torch.zeros(64, dtype=torch.float32, device=DEV)
    # T == 0: success, nothing written, pointers not needed
    B.lmoe_route_permute(0, 16, 4, None, None, 1.0, 1, None, None, 16, None, None, None, None, None, None, 0, None, 0)
    with pytest.raises(B.LmoeError) as ei:   # rows_cap too small
        B.lmoe_route_permute(2, 16, 4, f, None, 1.0, 1, z, f, 16, z, z, z, z, z, z, 16, None, 0)
    assert ei.value.status == B.LMOE_ERR_WORKSPACE
    with pytest.raises(B.LmoeError) as ei:   # K > E
        B.lmoe_route_permute(2, 4, 8, f, None, 1.0, 1, z, f, 16, z, z, z, z, z, z, 256, None, 0)
    assert ei.value.status == B.LMOE_ERR_INVALID_ARG


def test_permute_capacity_checks(B):
    ids = torch.zeros(4, 2, dtype=torch.int32, device=DEV)
    z = torch.zeros(64, dtype=torch.int32, device=DEV)
    from latent_moe_layer_sigmoid_amd.binding import LmoeError
    with pytest.raises(LmoeError) as ei:
        B.lmoe_permute(4, 8, 2, 16, ids, z, z, z, z, z, z, 16, None, 0)   # rows_cap too small
    assert ei.value.status == B.LMOE_ERR_WORKSPACE
    with pytest.raises(LmoeError) as ei:
        B.lmoe_permute(4, 8, 2, 24, ids, z, z, z, z, z, z, 192, None, 0)  # unsupported tile
    assert ei.value.status == B.LMOE_ERR_INVALID_ARG


# ------------------------------------------------------------------------- masked SituGLU

def test_situ_masked_full_shape(B):
    cfg = LI.ROUTE_MASKED
    logits, bias, _ = guarded_route_logits(cfg, seed=3)
    ids, _, _ = oracle.route(logits.double().numpy(), bias.double().numpy(), cfg.K, cfg.rsf)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    counts_t = torch.from_numpy(counts.astype(np.int32))
    inp = LI.make_masked_input(cfg, seed=3, counts=counts_t, device=DEV)
    out = torch.empty(cfg.E, cfg.T_max, cfg.d, dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(LI.BF16_SENTINEL - 65536)
    B.lmoe_situ_masked(cfg.E, cfg.T_max, cfg.d, B.LMOE_BF16, inp, counts_t.to(DEV), cfg.beta, cfg.linear_beta, out)
    torch.cuda.synchronize()
    got_bits = out.view(torch.int16).cpu().numpy().astype(np.int64) & 0xFFFF
    v = np.clip(counts, 0, cfg.T_max)
    pad = np.arange(cfg.T_max)[None, :] >= v[:, None]
    assert np.all(got_bits[pad] == LI.BF16_SENTINEL)          # padded rows bit-untouched
    ref = oracle.situ_masked(f64(inp), counts, cfg.beta, cfg.linear_beta, np.zeros((cfg.E, cfg.T_max, cfg.d)))
    valid = ~pad
    g = f64(out)[valid]
    r = ref[valid]
    assert norm_err(g, r) <= 1e-2
    ref_bits = (torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64) & 0xFFFF)
    assert bf16_ulp_diff(got_bits[valid], ref_bits) <= 2


def test_situ_masked_f32_and_clamps(B):
    E, Tm, d = 5, 7, 24
    rng = np.random.default_rng(0)
    inp = torch.from_numpy(rng.standard_normal((E, Tm, 2 * d)).astype(np.float32))
    counts = np.array([0, 3, 7, 11, -4], dtype=np.int32)
    out = torch.full((E, Tm, d), float("nan"), device=DEV)
    B.lmoe_situ_masked(E, Tm, d, B.LMOE_F32, inp.to(DEV), torch.from_numpy(counts).to(DEV), 0.7, 0.0, out)
    torch.cuda.synchronize()
    ref = oracle.situ_masked(inp.double().numpy(), counts, 0.7, 0.0, np.full((E, Tm, d), np.nan), dtype="f32")
    got = out.cpu().double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_allclose(got[ok], ref[ok], rtol=2e-5, atol=1e-6)


@pytest.mark.parametrize("linear_beta", [0.5, 0.0])
def test_situ_masked_f32_relative_small_arguments(B, linear_beta):
    """fp32 SituGLU element by element, relative error only: gate and up values spread
    log-uniformly over [1e-6, 4] in magnitude, so that tanh and sigmoid are evaluated near
    zero, where 1 - 2 / (exp(2x) + 1) alone would lose most of its relative accuracy; counts
    that end inside, at and past the 16-row chunks the kernel works in."""
    E, Tm, d = 6, 40, 64
    rng = np.random.default_rng(17)
    mag = 10.0 ** rng.uniform(-6, np.log10(4.0), (E, Tm, 2 * d))
    inp = torch.from_numpy((mag * rng.choice([-1.0, 1.0], mag.shape)).astype(np.float32))
    counts = np.array([0, 1, 16, 17, 33, 40], dtype=np.int32)
    out = torch.full((E, Tm, d), float("nan"), device=DEV)
    B.lmoe_situ_masked(E, Tm, d, B.LMOE_F32, inp.to(DEV), torch.from_numpy(counts).to(DEV), 1.0, linear_beta, out)
    torch.cuda.synchronize()
    ref = oracle.situ_masked(inp.double().numpy(), counts, 1.0, linear_beta, np.full((E, Tm, d), np.nan), dtype="f32")
    got = out.cpu().double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    rel = np.abs(got[ok] - ref[ok]) / np.abs(ref[ok])
    print(f"[situ f32] max relative error {rel.max():.3e}", flush=True)
    assert rel.max() <= 2e-6


# -------------------------------------------------------------------------- MXFP8 quant

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quant_mxfp8_bit_exact(B, dtype):
    rng = np.random.default_rng(9)
    rows, cols = 67, 2048
    v = rng.standard_normal((rows, cols)) * 10.0 ** rng.integers(-4, 4, (rows, 1))
    v[3, :32] = 0.0                              # all-zero block
    v[4, 32:64] = 1.0                            # power-of-two block
    v[5, 64:96] = 0.75
    v[5, 70] = 480.0                             # saturating element
    v[6, 96:128] = -1e-6                         # tiny block
    v[7, 0:32] *= 1e-30                          # very small exponent
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(v).to(td)
    codes = torch.zeros(rows, cols, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(rows, cols // 32, dtype=torch.uint8, device=DEV)
    B.lmoe_quant_mxfp8(rows, cols, B.LMOE_BF16 if dtype == "bf16" else B.LMOE_F32, x.to(DEV), codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.mxfp8_quantize(f64(x))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


# ------------------------------------------------------------------------- weight packing

def _pack_reference(w):
    """Packed layout from its definition (include/lmoe.h, lmoe_pack_weights), in numpy."""
    N, Kd = w.shape
    es = w.itemsize
    kch = 256 // es
    nch = Kd // kch
    v = 16 // es
    out = np.empty(N * Kd, dtype=w.dtype)
    for n16 in range(N // 16):
        for c in range(nch):
            blk = (n16 * nch + c) * (4096 // es)
            for q in range(4):
                for g in range(4):
                    for r in range(16):
                        k0 = c * kch + q * (kch // 4) + g * (kch // 16)
                        dst = blk + (q * 1024 + g * 256 + r * 16) // es
                        out[dst:dst + v] = w[n16 * 16 + r, k0:k0 + v]
    return out.reshape(N, Kd)


@pytest.mark.parametrize("N,Kd,dt", [(16, 128, "bf16"), (48, 384, "bf16"), (32, 64, "f32"), (16, 192, "f32")])
def test_pack_weights_layout(B, N, Kd, dt):
    rng = np.random.default_rng(N + Kd)
    if dt == "bf16":
        bits = rng.integers(0, 1 << 16, (3, N, Kd)).astype(np.uint16)
        src = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        src = torch.from_numpy(rng.standard_normal((3, N, Kd)).astype(np.float32)).to(DEV)
    got = B.packed(src)
    torch.cuda.synchronize()
    view = torch.int16 if dt == "bf16" else torch.int32
    g = got.view(view).cpu().numpy()
    s_np = src.view(view).cpu().numpy()
    for b in range(3):
        assert np.array_equal(g[b], _pack_reference(s_np[b]))


# ------------------------------------------------------------------------- dense linear

@pytest.mark.parametrize("M,N,Kd,dt,yt", [(1, 16, 128, "bf16", "f32"), (8, 896, 7168, "bf16", "f32"),
                                          (8, 2048, 7168, "bf16", "bf16"), (17, 48, 256, "bf16", "bf16"),
                                          (4, 16, 256, "f32", "f32"), (33, 128, 192, "f32", "f32"),
                                          (200, 64, 384, "bf16", "f32"), (300, 400, 640, "bf16", "bf16"),
                                          (256, 128, 128, "bf16", "f32"),
                                          # several column blocks per wave, partial last group
                                          (240, 17600, 384, "bf16", "bf16"), (200, 20240, 64, "f32", "f32")])
def test_linear_matches_oracle(B, M, N, Kd, dt, yt):
    rng = np.random.default_rng(M + N + Kd)
    td = torch.bfloat16 if dt == "bf16" else torch.float32
    x = torch.from_numpy(rng.standard_normal((M, Kd))).to(td)
    w = torch.from_numpy(rng.standard_normal((N, Kd)) / math.sqrt(Kd)).to(td)
    y = torch.empty(M, N, dtype=torch.float32 if yt == "f32" else torch.bfloat16, device=DEV)
    B.lmoe_linear(M, N, Kd, B.LMOE_BF16 if dt == "bf16" else B.LMOE_F32, x.to(DEV),
                  B.LMOE_BF16 if dt == "bf16" else B.LMOE_F32, B.packed(w.to(DEV)),
                  B.LMOE_F32 if yt == "f32" else B.LMOE_BF16, y)
    torch.cuda.synchronize()
    ref = oracle.round_to(oracle.linear(f64(x), f64(w)), yt)
    assert norm_err(f64(y), ref) <= (1e-5 if yt == "f32" else 8e-3)


# -------------------------------------------------------------------- grouped expert GEMMs

def _expert_case(B, T, E, K, L, d, tile_m, dt, seed, ids=None):
    rng = np.random.default_rng(seed)
    td = torch.bfloat16 if dt == "bf16" else torch.float32
    if ids is None:
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    w = rng.random((T, K)).astype(np.float32) + 0.1
    x = torch.from_numpy(rng.standard_normal((T, L))).to(td)
    W1 = torch.from_numpy(rng.standard_normal((E, 2 * d, L)) / math.sqrt(L)).to(td)
    W2 = torch.from_numpy(rng.standard_normal((E, L, d)) / math.sqrt(d)).to(td)
    perm = oracle.permute(ids, E, tile_m)
    rc = B.lmoe_permute_rows_cap(T, E, K, tile_m)
    i32 = lambda a, n: torch.from_numpy(np.concatenate([a, np.full(n - len(a), -1)]).astype(np.int32)).to(DEV)
    r2p = i32(perm["row_to_pair"], rc)
    te = torch.from_numpy(tile_expert_from_offsets(perm["tile_offsets"], tile_m, rc // tile_m).astype(np.int32)).to(DEV)
    return dict(ids=ids, w=w, x=x, W1=W1, W2=W2, perm=perm, rc=rc, r2p=r2p, te=te, td=td)


@pytest.mark.parametrize("T,E,K,L,d,tile_m,dt", [(4, 16, 4, 128, 64, 16, "f32"), (8, 64, 16, 2048, 512, 16, "bf16"),
                                                 (50, 32, 4, 256, 128, 32, "bf16"),
                                                 (300, 16, 2, 256, 128, 128, "bf16"),
                                                 (600, 64, 8, 1024, 256, 128, "bf16"),
                                                 # several column blocks per wave: FC2 (three) and FC1 (two)
                                                 (256, 64, 8, 2048, 128, 16, "bf16"),
                                                 (256, 128, 8, 256, 512, 16, "bf16")])
def test_fc1_fc2_grouped_match_oracle(B, T, E, K, L, d, tile_m, dt):
    _check_fc1_fc2(B, _expert_case(B, T, E, K, L, d, tile_m, dt, seed=T + E), T, E, K, L, d, tile_m, dt)


def test_fc1_fc2_tiled_padding_quarters(B):
    """128-row expert tiles whose last rows are padding: expert counts on both sides of
    every 32-row boundary, so that a tile's wavefronts compute two, one or none of their
    32-row quarters; two experts receive no pair."""
    counts = [1, 31, 32, 33, 63, 64, 65, 95, 0, 96, 97, 127, 128, 129, 160, 200, 256, 0]
    E, K, L, d, tile_m = len(counts), 1, 256, 128, 128
    ids = np.repeat(np.arange(E, dtype=np.int32), counts)
    np.random.default_rng(5).shuffle(ids)
    T = len(ids)
    c = _expert_case(B, T, E, K, L, d, tile_m, "bf16", seed=17, ids=ids.reshape(T, K))
    assert np.array_equal(np.diff(c["perm"]["offsets"]), counts)
    _check_fc1_fc2(B, c, T, E, K, L, d, tile_m, "bf16")


def _check_fc1_fc2(B, c, T, E, K, L, d, tile_m, dt):
    ldt = B.LMOE_BF16 if dt == "bf16" else B.LMOE_F32
    rc = c["rc"]
    sentinel = -12288.0   # exact in bf16 and fp32
    act = torch.full((rc, d), sentinel, dtype=c["td"], device=DEV)
    B.lmoe_fc1_situ(T, E, K, L, d, tile_m, ldt, c["x"].to(DEV), None, c["r2p"], c["te"], ldt, B.packed(c["W1"].to(DEV)), None,
                    1.0, 0.5, ldt, act, None, rc)
    torch.cuda.synchronize()
    r2p = c["perm"]["row_to_pair"]
    x64, W1_64, W2_64 = f64(c["x"]), f64(c["W1"]), f64(c["W2"])
    act64 = f64(act)
    ref_act = np.zeros((len(r2p), d))
    for r, p in enumerate(r2p):
        if p >= 0:
            e = c["ids"].reshape(-1)[p]
            h = oracle.linear(x64[p // K][None, :], W1_64[e])
            ref_act[r] = oracle.round_to(oracle.situ_glu_rows(h, 1.0, 0.5), dt)[0]
    valid = r2p >= 0
    assert norm_err(act64[:len(r2p)][valid], ref_act[valid]) <= 1e-2
    assert np.all(act64[:len(r2p)][~valid] == sentinel)        # pad rows never written
    assert np.all(act64[len(r2p):] == sentinel)
    # FC2 + combine on independently generated activation rows (pad rows left as garbage)
    rng = np.random.default_rng(T + 3)
    act_in = torch.from_numpy(rng.standard_normal((rc, d))).to(c["td"])
    z = torch.full((T, L), float("nan"), device=DEV)
    wsb = B.lmoe_fc2_workspace_bytes(T, K, L)
    ws = torch.empty(max(wsb // 4, 1), device=DEV)
    B.lmoe_fc2_combine(T, E, K, d, L, tile_m, ldt, act_in.to(DEV), None, c["r2p"], c["te"], ldt,
                       B.packed(c["W2"].to(DEV)), None, torch.from_numpy(c["w"]).to(DEV), B.LMOE_F32, z, rc, ws, wsb)
    torch.cuda.synchronize()
    a64 = f64(act_in)
    ref_z = np.zeros((T, L))
    p2r = c["perm"]["pair_to_row"]
    for t in range(T):
        for k in range(K):
            e = c["ids"][t, k]
            y = oracle.linear(a64[p2r[t * K + k]][None, :], W2_64[e])[0]
            ref_z[t] += c["w"][t, k].astype(np.float64) * y
    assert norm_err(f64(z), oracle.f32_round(ref_z)) <= 1e-4


def test_fc2_combine_wide_short_k(B):
    """FC2 with many short-K work items (the decode regime) over 33 column blocks of 64,
    the last one partial, against the oracle's weighted combine."""
    T, E, K, d, out_dim, tile_m = 256, 32, 8, 128, 2064, 16
    rng = np.random.default_rng(9)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    wts = rng.random((T, K)).astype(np.float32) + 0.1
    perm = oracle.permute(ids, E, tile_m)
    rc = B.lmoe_permute_rows_cap(T, E, K, tile_m)
    r2p = torch.from_numpy(np.concatenate([perm["row_to_pair"], np.full(rc - len(perm["row_to_pair"]), -1)])
                           .astype(np.int32)).to(DEV)
    te = torch.from_numpy(tile_expert_from_offsets(perm["tile_offsets"], tile_m, rc // tile_m).astype(np.int32)).to(DEV)
    act = torch.from_numpy(rng.standard_normal((rc, d))).to(torch.bfloat16)
    W2 = torch.from_numpy(rng.standard_normal((E, out_dim, d)) / math.sqrt(d)).to(torch.bfloat16)
    z = torch.full((T, out_dim), float("nan"), device=DEV)
    wsb = B.lmoe_fc2_workspace_bytes(T, K, out_dim)
    ws = torch.empty(max(wsb // 4, 1), device=DEV)
    B.lmoe_fc2_combine(T, E, K, d, out_dim, tile_m, B.LMOE_BF16, act.to(DEV), None, r2p, te, B.LMOE_BF16,
                       B.packed(W2.to(DEV)), None, torch.from_numpy(wts).to(DEV), B.LMOE_F32, z, rc, ws, wsb)
    torch.cuda.synchronize()
    a64, W2_64 = f64(act), f64(W2)
    ref = np.zeros((T, out_dim))
    p2r = perm["pair_to_row"]
    for t in range(T):
        for k in range(K):
            ref[t] += wts[t, k].astype(np.float64) * (W2_64[ids[t, k]] @ a64[p2r[t * K + k]])
    assert norm_err(f64(z), oracle.f32_round(ref)) <= 1e-4


@pytest.mark.parametrize("T,E,K,L,d,tile_m,dt", [(8, 64, 16, 2048, 512, 16, "bf16"), (4, 16, 4, 128, 64, 16, "f32"),
                                                 (300, 16, 2, 256, 128, 128, "bf16"), (5, 1, 1, 256, 128, 16, "bf16")])
def test_fc2_combine_norm_matches_two_calls_and_oracle(B, T, E, K, L, d, tile_m, dt):
    """FC2 + combine + RMSNorm in one call: z and the normalized latent are bit-identical
    to lmoe_fc2_combine followed by lmoe_tail's RMSNorm, and within tolerance of the
    oracle's combine and RMSNorm."""
    c = _expert_case(B, T, E, K, L, d, tile_m, dt, seed=T + E + 11)
    ldt = B.LMOE_BF16 if dt == "bf16" else B.LMOE_F32
    rc = c["rc"]
    dense = E == 1 and K == 1
    r2p, te = (None, None) if dense else (c["r2p"], c["te"])
    rcap = T if dense else rc
    rng = np.random.default_rng(T + 5)
    act_in = torch.from_numpy(rng.standard_normal((rcap, d))).to(c["td"]).to(DEV)
    W2p = B.packed(c["W2"].to(DEV))
    wts = torch.from_numpy(c["w"]).to(DEV)
    gamma = torch.from_numpy(rng.uniform(0.9, 1.1, L)).to(c["td"]).to(DEV)
    wsb = B.lmoe_fc2_workspace_bytes(T, K, L)
    ws = torch.empty(max(wsb // 4, 1), device=DEV)
    z1 = torch.full((T, L), float("nan"), device=DEV)
    B.lmoe_fc2_combine(T, E, K, d, L, tile_m, ldt, act_in, None, r2p, te, ldt, W2p, None, wts, B.LMOE_F32, z1, rcap,
                       ws, wsb)
    n1 = torch.empty(T, L, dtype=c["td"], device=DEV)
    out = torch.empty(T, 16, dtype=c["td"], device=DEV)
    w_up = B.packed(torch.zeros(16, L, dtype=c["td"], device=DEV))
    B.lmoe_tail(T, L, 16, z1, gamma, 1e-6, w_up, None, ldt, out, n1)
    z2 = torch.full((T, L), float("nan"), device=DEV)
    n2 = torch.full((T, L), float("nan"), dtype=c["td"], device=DEV)
    B.lmoe_fc2_combine_norm(T, E, K, d, L, tile_m, ldt, act_in, None, r2p, te, ldt, W2p, None, wts, z2, rcap, ws, wsb,
                            gamma, 1e-6, ldt, n2)
    torch.cuda.synchronize()
    assert torch.equal(z1.view(torch.int32), z2.view(torch.int32))
    assert torch.equal(n1.view(torch.int16) if dt == "bf16" else n1.view(torch.int32),
                       n2.view(torch.int16) if dt == "bf16" else n2.view(torch.int32))
    # oracle: combine of the expert products, then RMSNorm
    a64, W2_64 = f64(act_in), f64(c["W2"])
    p2r = np.arange(T) if dense else c["perm"]["pair_to_row"]
    ref_z = np.zeros((T, L))
    for t in range(T):
        for k in range(K):
            e = 0 if dense else c["ids"][t, k]
            y = oracle.linear(a64[p2r[t * K + k]][None, :], W2_64[e])[0]
            ref_z[t] += c["w"][t, k].astype(np.float64) * y
    ref_z = oracle.f32_round(ref_z)
    assert norm_err(f64(z2), ref_z) <= 1e-4
    assert norm_err(f64(n2), oracle.round_to(oracle.rmsnorm(ref_z, f64(gamma), 1e-6), dt)) <= 1e-2


# ------------------------------------------------------------------ MX (MXFP8 x MXFP4) experts

def _pack_mxfp4_reference(codes, scales):
    """Packed MXFP4 layout from its definition (include/lmoe.h, lmoe_pack_mxfp4_weights)."""
    N, half_k = codes.shape
    Kd = half_k * 2
    nst = Kd // 512
    pc = np.empty(N * Kd // 2, dtype=np.uint8)
    ps = np.empty(N * Kd // 32, dtype=np.uint8)
    for n16 in range(N // 16):
        for st in range(nst):
            blk = n16 * nst + st
            for q in range(4):
                for g in range(4):
                    for r in range(16):
                        b0 = (st * 512 + q * 128 + g * 32) // 2
                        dst = blk * 4096 + q * 1024 + g * 256 + r * 16
                        pc[dst:dst + 16] = codes[n16 * 16 + r, b0:b0 + 16]
                        ps[blk * 256 + (16 * g + r) * 4 + q] = scales[n16 * 16 + r, st * 16 + q * 4 + g]
    return pc.reshape(N, half_k), ps.reshape(N, Kd // 32)


def test_pack_mxfp4_layout(B):
    rng = np.random.default_rng(3)
    N, Kd = 32, 1024
    codes = rng.integers(0, 256, (2, N, Kd // 2)).astype(np.uint8)
    scales = rng.integers(0, 255, (2, N, Kd // 32)).astype(np.uint8)
    pc, ps = B.packed_mxfp4(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV))
    torch.cuda.synchronize()
    for b in range(2):
        rc, rs = _pack_mxfp4_reference(codes[b], scales[b])
        assert np.array_equal(pc[b].cpu().numpy(), rc)
        assert np.array_equal(ps[b].cpu().numpy(), rs)


def _mx_weights(rng, E, N, Kd):
    codes = rng.integers(0, 256, (E, N, Kd // 2)).astype(np.uint8)
    scales = rng.integers(118, 123, (E, N, Kd // 32)).astype(np.uint8)
    return codes, scales


@pytest.mark.parametrize("T,E,K,L,d,tile_m", [(24, 8, 4, 1024, 512, 16), (40, 16, 8, 512, 512, 32),
                                             (50, 8, 4, 512, 512, 64)])
def test_fc1_fc2_mx_match_oracle(B, T, E, K, L, d, tile_m):
    rng = np.random.default_rng(T + E)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    wts = (rng.random((T, K)) + 0.1).astype(np.float32)
    perm = oracle.permute(ids, E, tile_m)
    rc = B.lmoe_permute_rows_cap(T, E, K, tile_m)
    r2p = torch.from_numpy(np.concatenate([perm["row_to_pair"], np.full(rc - len(perm["row_to_pair"]), -1)])
                           .astype(np.int32)).to(DEV)
    te = torch.from_numpy(tile_expert_from_offsets(perm["tile_offsets"], tile_m, rc // tile_m).astype(np.int32)).to(DEV)
    # activations quantized by the oracle's codec (inputs never come from the GPU path)
    xq, xs = oracle.mxfp8_quantize(oracle.bf16_round(rng.standard_normal((T, L))))
    W1c, W1s = _mx_weights(rng, E, 2 * d, L)
    W2c, W2s = _mx_weights(rng, E, L, d)
    p1c, p1s = B.packed_mxfp4(torch.from_numpy(W1c).to(DEV), torch.from_numpy(W1s).to(DEV))
    p2c, p2s = B.packed_mxfp4(torch.from_numpy(W2c).to(DEV), torch.from_numpy(W2s).to(DEV))
    act = torch.full((rc, d), 0x55, dtype=torch.uint8, device=DEV)
    act_s = torch.full((rc, d // 32), 0x55, dtype=torch.uint8, device=DEV)
    B.lmoe_fc1_situ(T, E, K, L, d, tile_m, B.LMOE_MXFP8_E4M3, torch.from_numpy(xq).to(DEV),
                    torch.from_numpy(xs).to(DEV), r2p, te, B.LMOE_MXFP4_E2M1, p1c, p1s, 1.0, 0.0,
                    B.LMOE_MXFP8_E4M3, act, act_s, rc)
    torch.cuda.synchronize()
    x_hat = oracle.mxfp8_dequant(xq, xs)
    flat = ids.reshape(-1)
    r2p_np = perm["row_to_pair"]
    rows = np.nonzero(r2p_np >= 0)[0]
    got_c, got_s = act.cpu().numpy(), act_s.cpu().numpy()
    ref_c = np.zeros((len(rows), d), np.uint8)
    ref_s = np.zeros((len(rows), d // 32), np.uint8)
    for i, r in enumerate(rows):
        p = r2p_np[r]
        h = oracle.linear(x_hat[p // K][None, :], oracle.mxfp4_dequant(W1c[flat[p]], W1s[flat[p]]))
        a32 = oracle.f32_round(oracle.situ_glu_rows(h, 1.0, 0.0))
        ref_c[i], ref_s[i] = [v[0] for v in oracle.mxfp8_quantize(a32)]
    assert np.mean(got_c[rows] == ref_c) >= 0.99 and np.mean(got_s[rows] == ref_s) >= 0.99
    deq_g = oracle.mxfp8_dequant(got_c[rows], got_s[rows])
    deq_r = oracle.mxfp8_dequant(ref_c, ref_s)
    assert norm_err(deq_g, deq_r) <= 0.07                       # at most about one e4m3 step
    pad = np.nonzero(r2p_np < 0)[0]
    assert np.all(got_c[pad] == 0x55) and np.all(got_s[pad] == 0x55)   # pad rows never written
    # FC2 + combine on independently quantized activation rows
    aq, as_ = oracle.mxfp8_quantize(oracle.bf16_round(rng.standard_normal((rc, d))))
    z = torch.full((T, L), float("nan"), device=DEV)
    wsb = B.lmoe_fc2_workspace_bytes(T, K, L)
    ws = torch.empty(max(wsb // 4, 1), device=DEV)
    B.lmoe_fc2_combine(T, E, K, d, L, tile_m, B.LMOE_MXFP8_E4M3, torch.from_numpy(aq).to(DEV),
                       torch.from_numpy(as_).to(DEV), r2p, te, B.LMOE_MXFP4_E2M1, p2c, p2s,
                       torch.from_numpy(wts).to(DEV), B.LMOE_F32, z, rc, ws, wsb)
    torch.cuda.synchronize()
    a_hat = oracle.mxfp8_dequant(aq, as_)
    p2r = perm["pair_to_row"]
    ref_z = np.zeros((T, L))
    for t in range(T):
        for k in range(K):
            e = ids[t, k]
            y = oracle.linear(a_hat[p2r[t * K + k]][None, :], oracle.mxfp4_dequant(W2c[e], W2s[e]))[0]
            ref_z[t] += wts[t, k].astype(np.float64) * y
    assert norm_err(f64(z), oracle.f32_round(ref_z)) <= 1e-4


# output widths of 1, 2, 7, 9 and 32 blocks of 64 columns: a wavefront that walks several
# column blocks also meets a row tile's last, shorter run of blocks (or none); K = 1 stores
# the token rows directly
@pytest.mark.parametrize("T,E,K,d,out_dim,tile_m", [(40, 16, 8, 512, 576, 32), (24, 8, 4, 512, 448, 16),
                                                    (30, 8, 4, 1024, 64, 32), (20, 4, 1, 512, 128, 32),
                                                    (70, 4, 2, 512, 2048, 32)])
def test_fc2_mx_column_block_runs(B, T, E, K, d, out_dim, tile_m):
    rng = np.random.default_rng(T + out_dim)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    wts = (rng.random((T, K)) + 0.1).astype(np.float32)
    perm = oracle.permute(ids, E, tile_m)
    rc = B.lmoe_permute_rows_cap(T, E, K, tile_m)
    r2p = torch.from_numpy(np.concatenate([perm["row_to_pair"], np.full(rc - len(perm["row_to_pair"]), -1)])
                           .astype(np.int32)).to(DEV)
    te = torch.from_numpy(tile_expert_from_offsets(perm["tile_offsets"], tile_m, rc // tile_m).astype(np.int32)).to(DEV)
    W2c, W2s = _mx_weights(rng, E, out_dim, d)
    p2c, p2s = B.packed_mxfp4(torch.from_numpy(W2c).to(DEV), torch.from_numpy(W2s).to(DEV))
    aq, as_ = oracle.mxfp8_quantize(oracle.bf16_round(rng.standard_normal((rc, d))))
    z = torch.full((T, out_dim), float("nan"), device=DEV)
    wsb = B.lmoe_fc2_workspace_bytes(T, K, out_dim)
    ws = torch.empty(max(wsb // 4, 1), device=DEV)
    B.lmoe_fc2_combine(T, E, K, d, out_dim, tile_m, B.LMOE_MXFP8_E4M3, torch.from_numpy(aq).to(DEV),
                       torch.from_numpy(as_).to(DEV), r2p, te, B.LMOE_MXFP4_E2M1, p2c, p2s,
                       torch.from_numpy(wts).to(DEV), B.LMOE_F32, z, rc, ws, wsb)
    torch.cuda.synchronize()
    a_hat = oracle.mxfp8_dequant(aq, as_)
    p2r = perm["pair_to_row"]
    ref_z = np.zeros((T, out_dim))
    for t in range(T):
        for k in range(K):
            e = ids[t, k]
            y = oracle.linear(a_hat[p2r[t * K + k]][None, :], oracle.mxfp4_dequant(W2c[e], W2s[e]))[0]
            ref_z[t] += wts[t, k].astype(np.float64) * y
    assert norm_err(f64(z), oracle.f32_round(ref_z)) <= 1e-4


@pytest.mark.parametrize("max_waves", [0, 512, 256, 100, 64])
def test_fc1_situ_capped_matches_fc1_situ(B, max_waves):
    """The width-bounded FC1 against the oracle and against lmoe_fc1_situ: the shared
    expert's decode shape in dense mode, and a grouped decode-sized call. With fewer
    wavefronts K is split over fewer partial sums (another fp32 summation order), so the
    two calls agree bit for bit only at max_waves == 0."""
    rng = np.random.default_rng(7 + max_waves)
    T, H, I = 8, 7168, 4096
    X = torch.from_numpy(rng.standard_normal((T, H))).to(torch.bfloat16).to(DEV)
    Ws = torch.from_numpy(rng.standard_normal((2 * I, H)) / math.sqrt(H)).to(torch.bfloat16)
    W = B.packed(Ws.to(DEV))
    ref = torch.full((T, I), float("nan"), dtype=torch.bfloat16, device=DEV)
    got = torch.full_like(ref, float("nan"))
    B.lmoe_fc1_situ(T, 1, 1, H, I, 16, B.LMOE_BF16, X, None, None, None, B.LMOE_BF16, W, None, 1.0, 0.5,
                    B.LMOE_BF16, ref, None, T)
    B.lmoe_fc1_situ_capped(T, 1, 1, H, I, 16, B.LMOE_BF16, X, None, None, None, B.LMOE_BF16, W, None, 1.0, 0.5,
                           B.LMOE_BF16, got, None, T, max_waves)
    torch.cuda.synchronize()
    assert not torch.isnan(got.float()).any()
    ref64 = oracle.round_to(oracle.situ_glu_rows(oracle.linear(f64(X.cpu()), f64(Ws)), 1.0, 0.5),
                            "bf16")
    assert norm_err(f64(got), ref64) <= 1e-2
    if max_waves == 0:
        assert torch.equal(got, ref)
    else:
        assert norm_err(f64(got), f64(ref)) <= 1e-2      # one bf16 ulp is up to 2^-7 of the max
    # grouped: 8 tokens, 64 experts, top-16, tile 16
    c = _expert_case(B, 8, 64, 16, 2048, 512, 16, "bf16", seed=3)
    W1 = B.packed(c["W1"].to(DEV))
    acts = []
    for capped in (False, True):
        act = torch.full((c["rc"], 512), -12288.0, dtype=torch.bfloat16, device=DEV)
        args = (8, 64, 16, 2048, 512, 16, B.LMOE_BF16, c["x"].to(DEV), None, c["r2p"], c["te"], B.LMOE_BF16, W1,
                None, 1.0, 0.5, B.LMOE_BF16, act, None, c["rc"])
        if capped:
            B.lmoe_fc1_situ_capped(*args, max_waves)
        else:
            B.lmoe_fc1_situ(*args)
        acts.append(act)
    torch.cuda.synchronize()
    valid = torch.from_numpy(c["perm"]["row_to_pair"] >= 0)
    n = len(valid)
    a0, a1 = f64(acts[0][:n][valid.to(DEV)]), f64(acts[1][:n][valid.to(DEV)])
    assert norm_err(a1, a0) <= 1e-2
    assert torch.equal(acts[0][:n][~valid.to(DEV)], acts[1][:n][~valid.to(DEV)])   # pad rows untouched


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_dense_mode_shared_expert(B, dt):
    rng = np.random.default_rng(4)
    T, H, I = 8, 256, 128
    td = torch.bfloat16 if dt == "bf16" else torch.float32
    ldt = B.LMOE_BF16 if dt == "bf16" else B.LMOE_F32
    X = torch.from_numpy(rng.standard_normal((T, H))).to(td)
    Ws1 = torch.from_numpy(rng.standard_normal((2 * I, H)) / 16).to(td)
    Ws2 = torch.from_numpy(rng.standard_normal((H, I)) / 11).to(td)
    a = torch.empty(T, I, dtype=td, device=DEV)
    sh = torch.empty(T, H, dtype=td, device=DEV)
    B.lmoe_fc1_situ(T, 1, 1, H, I, 16, ldt, X.to(DEV), None, None, None, ldt, B.packed(Ws1.to(DEV)), None, 1.0, 0.0,
                    ldt, a, None, T)
    B.lmoe_fc2_combine(T, 1, 1, I, H, 16, ldt, a, None, None, None, ldt, B.packed(Ws2.to(DEV)), None, None, ldt, sh, T,
                       None, 0)
    torch.cuda.synchronize()
    ref = oracle.shared_expert(f64(X), f64(Ws1), f64(Ws2), 1.0, 0.0, dt)
    assert norm_err(f64(sh), ref) <= 1e-2


# M = 260, 300, 340, 480: the last 128-row tile holds 4, 44, 84 and 96 rows
@pytest.mark.parametrize("M,Kd,dt", [(8, 7168, "bf16"), (3, 256, "f32"), (37, 384, "bf16"), (260, 512, "bf16"),
                                     (300, 256, "bf16"), (340, 512, "bf16"), (480, 256, "bf16")])
def test_linear_multi_matches_oracle(B, M, Kd, dt):
    rng = np.random.default_rng(M + Kd)
    td = torch.bfloat16 if dt == "bf16" else torch.float32
    ldt = B.LMOE_BF16 if dt == "bf16" else B.LMOE_F32
    N = [48, 128, 64]
    x = torch.from_numpy(rng.standard_normal((M, Kd))).to(td)
    ws = [torch.from_numpy(rng.standard_normal((n * (2 if i == 2 else 1), Kd)) / math.sqrt(Kd)).to(td)
          for i, n in enumerate(N)]
    ys = [torch.empty(M, N[0], device=DEV), torch.empty(M, N[1], dtype=td, device=DEV),
          torch.empty(M, N[2], dtype=td, device=DEV)]
    B.lmoe_linear_multi(M, Kd, ldt, x.to(DEV), 3, N, [B.packed(w.to(DEV)) for w in ws], [B.LMOE_F32, ldt, ldt], ys,
                        [0, 0, 1], 1.0, 0.5)
    torch.cuda.synchronize()
    x64 = f64(x)
    assert norm_err(f64(ys[0]), oracle.f32_round(oracle.linear(x64, f64(ws[0])))) <= 1e-5
    assert norm_err(f64(ys[1]), oracle.round_to(oracle.linear(x64, f64(ws[1])), dt)) <= 8e-3
    ref2 = oracle.round_to(oracle.situ_glu_rows(oracle.linear(x64, f64(ws[2])), 1.0, 0.5), dt)
    assert norm_err(f64(ys[2]), ref2) <= 1e-2


@pytest.mark.parametrize("M,Kd,N,situ", [(1024, 7168, [896, 2048], [0, 0]), (260, 2048, [48, 128, 64], [0, 0, 1]),
                                          (384, 1024, [400], [1])])
def test_linear_multi_split_k(B, M, Kd, N, situ):
    """Split-K of the tiled kernel (caller workspace): against the oracle, and within
    rounding of the unsplit call."""
    rng = np.random.default_rng(M + Kd + len(N))
    x = torch.from_numpy(rng.standard_normal((M, Kd))).to(torch.bfloat16)
    ws = [torch.from_numpy(rng.standard_normal((n * (2 if si else 1), Kd)) / math.sqrt(Kd)).to(torch.bfloat16)
          for n, si in zip(N, situ)]
    yt = [B.LMOE_F32 if i == 0 else B.LMOE_BF16 for i in range(len(N))]
    mk = lambda: [torch.full((M, n), float("nan"), dtype=torch.float32 if i == 0 else torch.bfloat16, device=DEV)
                  for i, n in enumerate(N)]
    wsb = B.lmoe_linear_multi_workspace_bytes(M, Kd, B.LMOE_BF16, len(N), N, situ)
    assert wsb > 0                      # these shapes split
    wp = [B.packed(w.to(DEV)) for w in ws]
    xd = x.to(DEV)
    y_split, y_plain = mk(), mk()
    work = torch.empty(wsb // 4, device=DEV)
    B.lmoe_linear_multi_ws(M, Kd, B.LMOE_BF16, xd, len(N), N, wp, yt, y_split, situ, 1.0, 0.5, work, wsb)
    B.lmoe_linear_multi(M, Kd, B.LMOE_BF16, xd, len(N), N, wp, yt, y_plain, situ, 1.0, 0.5)
    with pytest.raises(B.LmoeError) as ei:
        B.lmoe_linear_multi_ws(M, Kd, B.LMOE_BF16, xd, len(N), N, wp, yt, y_split, situ, 1.0, 0.5, work, wsb - 4)
    assert ei.value.status == B.LMOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    x64 = f64(x)
    for i, (n, si) in enumerate(zip(N, situ)):
        h = oracle.linear(x64, f64(ws[i]))
        ref = oracle.situ_glu_rows(h, 1.0, 0.5) if si else h
        ref = oracle.f32_round(ref) if i == 0 else oracle.round_to(ref, "bf16")
        tol = 1e-5 if i == 0 else 1e-2
        assert norm_err(f64(y_split[i]), ref) <= tol
        assert norm_err(f64(y_split[i]), f64(y_plain[i])) <= tol


@pytest.mark.parametrize("T,L,H,I,dt", [(8, 2048, 7168, 4096, "bf16"), (4, 128, 256, 128, "f32"),
                                        (21, 256, 512, 384, "bf16"), (300, 256, 400, 384, "bf16")])
def test_tail_shared_matches_oracle(B, T, L, H, I, dt):
    rng = np.random.default_rng(T + L + I)
    td = torch.bfloat16 if dt == "bf16" else torch.float32
    ldt = B.LMOE_BF16 if dt == "bf16" else B.LMOE_F32
    z = torch.from_numpy(rng.standard_normal((T, L)) * 0.3).float()
    gamma = torch.from_numpy(rng.uniform(0.9, 1.1, L)).to(td)
    Wup = torch.from_numpy(rng.standard_normal((H, L)) / math.sqrt(L)).to(td)
    a_s = torch.from_numpy(rng.standard_normal((T, I))).to(td)
    Ws2 = torch.from_numpy(rng.standard_normal((H, I)) / math.sqrt(I)).to(td)
    out = torch.empty(T, H, dtype=td, device=DEV)
    n = torch.empty(T, L, dtype=td, device=DEV)
    B.lmoe_tail_shared(T, L, H, I, z.to(DEV), gamma.to(DEV), 1e-6, B.packed(Wup.to(DEV)), a_s.to(DEV),
                       B.packed(Ws2.to(DEV)), ldt, out, n)
    torch.cuda.synchronize()
    sh = oracle.round_to(oracle.linear(f64(a_s), f64(Ws2)), dt)
    rn, rout = oracle.tail(f64(z), f64(gamma), 1e-6, f64(Wup), sh, dt)
    assert norm_err(f64(n), rn) <= 1e-2
    assert norm_err(f64(out), rout) <= 1e-2


@pytest.mark.parametrize("T,L,H,I,c1", [(1024, 2048, 7168, 4096, 0), (300, 512, 400, 1280, 0),
                                         (300, 512, 400, 1536, 0), (8192, 2048, 7168, 4096, 6144),
                                         (2048, 512, 8704, 1536, 8192), (8192, 512, 7040, 512, 6144)])
def test_tail_shared_split_k_matches_oracle(B, T, L, H, I, c1):
    # the token-heavy fused tail with too few output tiles for the CUs: split-K slices over
    # both K phases, against the oracle and against the unsplit call. Slices of 32-wide
    # steps: 192 in 2 (the phase boundary at step 128 inside the second slice), 56 in 3
    # (boundary 40 inside the third), 64 in 4 (boundary 48 at the start of the fourth).
    # c1 > 0: tiles past whole rounds of the CUs (64 x 14 = 3.5 rounds; 16 x 17 = 272 tiles)
    # -- columns [0, c1) in one full-K launch, bit-identical to the unsplit call, the rest
    # split into 2 (of 192 or 32 steps) or 4 (of 64 steps) slices in a second launch; H =
    # 7040 leaves a last block of 384 columns in the split launch
    rng = np.random.default_rng(T + 7 * L + I)
    td = torch.bfloat16
    z = torch.from_numpy(rng.standard_normal((T, L)) * 0.3).float()
    gamma = torch.from_numpy(rng.uniform(0.9, 1.1, L)).to(td)
    Wup = torch.from_numpy(rng.standard_normal((H, L)) / math.sqrt(L)).to(td)
    a_s = torch.from_numpy(rng.standard_normal((T, I))).to(td)
    Ws2 = torch.from_numpy(rng.standard_normal((H, I)) / math.sqrt(I)).to(td)
    wsb = B.lmoe_tail_shared_workspace_bytes(T, L, H, I, B.LMOE_BF16)
    assert wsb > 0              # 8 x 14 or 3 x 1 tiles on 256 CUs: split
    ws = torch.empty(max(wsb // 4, 1), dtype=torch.float32, device=DEV)
    args = (T, L, H, I, z.to(DEV), gamma.to(DEV), 1e-6, B.packed(Wup.to(DEV)), a_s.to(DEV), B.packed(Ws2.to(DEV)),
            B.LMOE_BF16)
    out, n = torch.empty(T, H, dtype=td, device=DEV), torch.empty(T, L, dtype=td, device=DEV)
    B.lmoe_tail_shared_ws(*args, out, n, ws, wsb)
    out1, n1 = torch.empty(T, H, dtype=td, device=DEV), torch.empty(T, L, dtype=td, device=DEV)
    B.lmoe_tail_shared(*args, out1, n1)
    if wsb > 0:
        with pytest.raises(B.LmoeError) as ei:
            B.lmoe_tail_shared_ws(*args, out1, n1, ws, wsb - 4)
        assert ei.value.status == B.LMOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    sel = np.arange(T) if T <= 300 else np.array([0, 1, T // 2 - 1, T - 2, T - 1])
    sh = oracle.round_to(oracle.linear(f64(a_s)[sel], f64(Ws2)), "bf16")
    rn, rout = oracle.tail(f64(z)[sel], f64(gamma), 1e-6, f64(Wup), sh, "bf16")
    assert norm_err(f64(n)[sel], rn) <= 1e-2
    assert norm_err(f64(out)[sel], rout) <= 1e-2
    assert norm_err(f64(out), f64(out1)) <= 1e-2
    if c1:
        assert torch.equal(out[:, :c1], out1[:, :c1])
        assert norm_err(f64(out)[:, c1:], f64(out1)[:, c1:]) <= 1e-2


# ------------------------------------------------------------------------------- tail

@pytest.mark.parametrize("T,L,H,dt,alias", [(8, 2048, 7168, "bf16", False), (4, 128, 256, "f32", True),
                                            (33, 256, 512, "bf16", True), (260, 384, 272, "bf16", True)])
def test_tail_matches_oracle(B, T, L, H, dt, alias):
    rng = np.random.default_rng(T + L)
    td = torch.bfloat16 if dt == "bf16" else torch.float32
    ldt = B.LMOE_BF16 if dt == "bf16" else B.LMOE_F32
    z = torch.from_numpy(rng.standard_normal((T, L)) * 0.3).float()
    gamma = torch.from_numpy(rng.uniform(0.9, 1.1, L)).to(td)
    Wup = torch.from_numpy(rng.standard_normal((H, L)) / math.sqrt(L)).to(td)
    sh = torch.from_numpy(rng.standard_normal((T, H))).to(td)
    sh_d = sh.to(DEV)
    out = sh_d if alias else torch.empty(T, H, dtype=td, device=DEV)
    n = torch.empty(T, L, dtype=td, device=DEV)
    B.lmoe_tail(T, L, H, z.to(DEV), gamma.to(DEV), 1e-6, B.packed(Wup.to(DEV)), sh_d, ldt, out, n)
    torch.cuda.synchronize()
    rn, rout = oracle.tail(f64(z), f64(gamma), 1e-6, f64(Wup), f64(sh), dt)
    assert norm_err(f64(n), rn) <= 1e-2
    assert norm_err(f64(out), rout) <= 1e-2
