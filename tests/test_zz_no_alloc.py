"""lmoe_permute_noalloc (the permutation for callers that cannot allocate: its per-block
counts live in the library's fixed device scratch) against lmoe_permute with a
caller workspace, through the C ABI: bit-identical outputs on two calls in a row, the
second with a smaller input, and the size limit rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def B():
    from latent_moe_layer_sigmoid_amd import binding
    binding.lib()
    return binding


def _ids(T, E, K, seed, skew):
    rng = np.random.default_rng(seed)
    p = np.exp(rng.standard_normal(E) * skew)
    p /= p.sum()
    return np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def _outputs(B, T, E, K, tile_m, fill):
    rc = B.lmoe_permute_rows_cap(T, E, K, tile_m)
    i32 = dict(dtype=torch.int32, device=DEV)
    return rc, dict(counts=torch.full((E,), fill, **i32), offsets=torch.full((E + 1,), fill, **i32),
                    tile_offsets=torch.full((E + 1,), fill, **i32), row_to_pair=torch.full((rc,), fill, **i32),
                    tile_expert=torch.full((rc // tile_m,), fill, **i32),
                    pair_to_row=torch.full((T * K,), fill, **i32))


def _both(B, ids_np, E, tile_m):
    T, K = ids_np.shape
    ids = torch.from_numpy(ids_np).to(DEV)
    rc, ref = _outputs(B, T, E, K, tile_m, -9)
    wsb = B.lmoe_permute_workspace_bytes(T, E, K)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=DEV)
    B.lmoe_permute(T, E, K, tile_m, ids, ref["counts"], ref["offsets"], ref["tile_offsets"], ref["row_to_pair"],
                   ref["tile_expert"], ref["pair_to_row"], rc, ws, wsb)
    _, got = _outputs(B, T, E, K, tile_m, -9)
    B.lmoe_permute_noalloc(T, E, K, tile_m, ids, got["counts"], got["offsets"], got["tile_offsets"],
                           got["row_to_pair"], got["tile_expert"], got["pair_to_row"], rc)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in ref.items()}, {k: v.cpu().numpy() for k, v in got.items()}


def _check_equal(ref, got, T, K):
    for k in ref:
        assert np.array_equal(ref[k], got[k]), k
    assert np.array_equal(got["row_to_pair"][got["pair_to_row"]], np.arange(T * K))


def test_noalloc_matches_workspace_call_twice_shrinking(B):
    E, K = 896, 16
    # first call: the prefill shape (128 blocks of pairs, 128-row tiles, skewed load)
    ref, got = _both(B, _ids(8192, E, K, 11, 1.0), E, 128)
    _check_equal(ref, got, 8192, K)
    # second call, smaller (45 blocks, 16-row tiles): the scratch keeps the first call's
    # counts, and none of them may leak into this one
    ref, got = _both(B, _ids(2900, E, K, 12, 0.5), E, 16)
    _check_equal(ref, got, 2900, K)
    # and a single-block batch, which needs no scratch
    ref, got = _both(B, _ids(8, E, K, 13, 0.0), E, 16)
    _check_equal(ref, got, 8, K)


def test_noalloc_rejects_more_than_its_scratch(B):
    E, K, tile_m = 1024, 64, 16
    limit = B.lmoe_permute_noalloc_max_bytes()
    assert limit == 1 << 20
    # ceil(T*K / 1024) * E * 4 bytes of counts: 5000 * 64 pairs -> 313 blocks -> 1.28 MB
    T = 5000
    assert (T * K + 1023) // 1024 * E * 4 > limit
    rc, o = _outputs(B, T, E, K, tile_m, -9)
    ids = torch.zeros(T, K, dtype=torch.int32, device=DEV)
    with pytest.raises(B.LmoeError) as ei:
        B.lmoe_permute_noalloc(T, E, K, tile_m, ids, o["counts"], o["offsets"], o["tile_offsets"],
                               o["row_to_pair"], o["tile_expert"], o["pair_to_row"], rc)
    assert ei.value.status == B.LMOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(o["counts"].min()) == -9 and int(o["counts"].max()) == -9   # nothing was enqueued
