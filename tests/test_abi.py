"""The C ABI without a GPU: liblmoe.so loads, exports every entry point include/lmoe.h
declares with the argument counts the Python binding uses, and rejects invalid calls
with the documented status codes before touching any HIP API."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmoe.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    funcs = {}
    for m in re.finditer(r"(?:lmoe_status|size_t|int|void|const char\s*\*)\s+(lmoe_\w+)\s*\(([^)]*)\)\s*;", src):
        args = m.group(2).strip()
        funcs[m.group(1)] = 0 if args in ("", "void") else len(args.split(","))
    return funcs


@pytest.fixture(scope="module")
def B():
    from latent_moe_layer_sigmoid_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from latent_moe_layer_sigmoid_amd.build_lib import build
        build()
    binding.lib()
    return binding


def test_header_declares_the_boundary():
    f = header_functions()
    for name in ("lmoe_route", "lmoe_permute", "lmoe_fc1_situ", "lmoe_fc2_combine", "lmoe_tail", "lmoe_linear",
                 "lmoe_situ_masked", "lmoe_quant_mxfp8"):
        assert name in f


def test_every_declared_symbol_is_exported_and_bound(B):
    lib = ctypes.CDLL(B.LIB_PATH)
    sigs = {n: a for n, _, a in B.SIGNATURES}
    for name, nargs in header_functions().items():
        assert hasattr(lib, name), name
        assert name in sigs, f"{name} missing from the Python binding"
        assert len(sigs[name]) == nargs, f"{name}: header has {nargs} args, binding {len(sigs[name])}"
    assert set(sigs) == set(header_functions())


def test_version_and_status_strings(B):
    assert B.lmoe_abi_version() == 1
    for s in range(5):
        assert B.lmoe_status_string(s)


def test_invalid_calls_are_rejected_without_a_gpu(B):
    L = B.lib()
    P = 0x1000   # never dereferenced: every call below fails validation first
    # route: K > E, K > 64, E too large
    assert L.lmoe_route(4, 8, 9, P, None, 1.0, 1, P, P, None) == B.LMOE_ERR_INVALID_ARG
    assert L.lmoe_route(4, 100, 65, P, None, 1.0, 1, P, P, None) == B.LMOE_ERR_INVALID_ARG
    assert L.lmoe_route(4, 2048, 16, P, None, 1.0, 1, P, P, None) == B.LMOE_ERR_UNSUPPORTED
    assert L.lmoe_route(4, 64, 4, None, None, 1.0, 1, P, P, None) == B.LMOE_ERR_INVALID_ARG
    assert L.lmoe_route(0, 64, 4, None, None, 1.0, 1, None, None, None) == B.LMOE_OK   # T == 0
    # permute: bad tile, capacity, workspace
    assert L.lmoe_permute(8, 64, 4, 24, P, P, P, P, P, P, P, 1024, P, 1 << 20, None) == B.LMOE_ERR_INVALID_ARG
    cap = B.lmoe_permute_rows_cap(8, 64, 4, 16)
    assert cap == 32 + 32 * 15
    assert L.lmoe_permute(8, 64, 4, 16, P, P, P, P, P, P, P, cap - 16, None, 0, None) == B.LMOE_ERR_WORKSPACE
    assert B.lmoe_permute_workspace_bytes(8, 64, 4) == 0
    assert B.lmoe_permute_workspace_bytes(8192, 896, 16) == 128 * 896 * 4
    # fused tail workspace (fp32 split-K slices, 128 x 512 tiles, 256 CUs): 8 x 14 tiles, two
    # slices of every column; 32 x 14 = 1.75 rounds, no split; 64 x 14 = 3.5 rounds, the last
    # 1024 columns (128 tiles) in two slices; 16 x 17 tiles, the last 512 columns in four
    assert B.lmoe_tail_shared_workspace_bytes(1024, 2048, 7168, 4096, B.LMOE_BF16) == 2 * 1024 * 7168 * 4
    assert B.lmoe_tail_shared_workspace_bytes(4096, 2048, 7168, 4096, B.LMOE_BF16) == 0
    assert B.lmoe_tail_shared_workspace_bytes(8192, 2048, 7168, 4096, B.LMOE_BF16) == 2 * 8192 * 1024 * 4
    assert B.lmoe_tail_shared_workspace_bytes(2048, 512, 8704, 1536, B.LMOE_BF16) == 4 * 2048 * 512 * 4
    assert B.lmoe_tail_shared_workspace_bytes(8192, 512, 7040, 512, B.LMOE_BF16) == 2 * 8192 * 896 * 4
    assert B.lmoe_tail_shared_workspace_bytes(8, 2048, 7168, 4096, B.LMOE_BF16) == 0   # few tokens: no tiled path
    big_cap = B.lmoe_permute_rows_cap(8192, 896, 16, 128)
    assert L.lmoe_permute(8192, 896, 16, 128, P, P, P, P, P, P, P, big_cap, None, 0, None) == B.LMOE_ERR_WORKSPACE
    # fc1: beta required and positive; mismatched dtypes; unsupported K dim
    cap = B.lmoe_permute_rows_cap(4, 16, 4, 16)
    for beta in (0.0, -1.0, float("nan"), float("inf")):
        assert L.lmoe_fc1_situ(4, 16, 4, 128, 64, 16, B.LMOE_F32, P, None, P, P, B.LMOE_F32, P, None, beta, 0.0,
                               B.LMOE_F32, P, None, cap, None) == B.LMOE_ERR_INVALID_ARG
    assert L.lmoe_fc1_situ(4, 16, 4, 128, 64, 16, B.LMOE_F32, P, None, P, P, B.LMOE_BF16, P, None, 1.0, 0.0,
                           B.LMOE_F32, P, None, cap, None) == B.LMOE_ERR_INVALID_ARG
    assert L.lmoe_fc1_situ(4, 16, 4, 100, 64, 16, B.LMOE_BF16, P, None, P, P, B.LMOE_BF16, P, None, 1.0, 0.0,
                           B.LMOE_BF16, P, None, cap, None) == B.LMOE_ERR_UNSUPPORTED
    # fc1 with a wave bound: the same checks, and the bound must not be negative
    assert L.lmoe_fc1_situ_capped(4, 16, 4, 128, 64, 16, B.LMOE_F32, P, None, P, P, B.LMOE_F32, P, None, 0.0, 0.0,
                                  B.LMOE_F32, P, None, cap, 512, None) == B.LMOE_ERR_INVALID_ARG
    assert L.lmoe_fc1_situ_capped(4, 1, 1, 128, 64, 16, B.LMOE_F32, P, None, None, None, B.LMOE_F32, P, None, 1.0,
                                  0.0, B.LMOE_F32, P, None, 4, -1, None) == B.LMOE_ERR_INVALID_ARG
    assert L.lmoe_fc1_situ_capped(0, 1, 1, 128, 64, 16, B.LMOE_F32, None, None, None, None, B.LMOE_F32, None, None,
                                  1.0, 0.0, B.LMOE_F32, None, None, 0, 512, None) == B.LMOE_OK   # T == 0
    # fc1 dense mode needs E == K == 1
    assert L.lmoe_fc1_situ(4, 2, 1, 128, 64, 16, B.LMOE_F32, P, None, None, None, B.LMOE_F32, P, None, 1.0, 0.0,
                           B.LMOE_F32, P, None, 4, None) == B.LMOE_ERR_INVALID_ARG
    # fc2: workspace too small for K > 1
    assert L.lmoe_fc2_combine(4, 16, 4, 64, 128, 16, B.LMOE_F32, P, None, P, P, B.LMOE_F32, P, None, P,
                              B.LMOE_F32, P, cap, P, 16, None) == B.LMOE_ERR_WORKSPACE
    assert B.lmoe_fc2_workspace_bytes(4, 4, 128) == 4 * 4 * 128 * 4
    # tail: eps < 0, bad dtype
    assert L.lmoe_tail(4, 128, 256, P, None, -1.0, P, None, B.LMOE_F32, P, P, None) == B.LMOE_ERR_INVALID_ARG
    assert L.lmoe_tail(4, 128, 256, P, None, 1e-6, P, None, B.LMOE_MXFP8_E4M3, P, P, None) == B.LMOE_ERR_INVALID_ARG
    # masked SituGLU: d % 8
    assert L.lmoe_situ_masked(4, 8, 12, B.LMOE_BF16, P, P, 1.0, 0.5, P, None) == B.LMOE_ERR_UNSUPPORTED
    assert L.lmoe_situ_masked(4, 8, 16, B.LMOE_BF16, P, P, 0.0, 0.5, P, None) == B.LMOE_ERR_INVALID_ARG
    # quant: cols % 32
    assert L.lmoe_quant_mxfp8(4, 48, B.LMOE_BF16, P, P, P, None) == B.LMOE_ERR_UNSUPPORTED
    # linear: N % 16, dtype mismatch
    assert L.lmoe_linear(4, 20, 128, B.LMOE_BF16, P, B.LMOE_BF16, P, B.LMOE_F32, P, None) == B.LMOE_ERR_UNSUPPORTED
    assert L.lmoe_linear(4, 32, 128, B.LMOE_BF16, P, B.LMOE_F32, P, B.LMOE_F32, P, None) == B.LMOE_ERR_INVALID_ARG


def test_layer_descriptions_are_checked_without_a_gpu(B):
    """lmoe_layer_create rejects a bad description before any HIP call: its own pointer
    and size checks, then the zero-token calls of every step (which touch no HIP API)."""
    import ctypes
    assert ctypes.sizeof(B.LayerDesc) == B.lmoe_layer_desc_bytes()
    L = B.lib()
    P = 0x1000   # never dereferenced

    def desc(**over):
        d = B.LayerDesc()
        d.T, d.H, d.L, d.E, d.K, d.d, d.I, d.tile_m = 8, 7168, 2048, 896, 16, 512, 4096, 16
        d.dtype, d.routing, d.n_group, d.topk_group = B.LMOE_BF16, B.LMOE_ROUTE_SIGMOID, 1, 1
        d.beta, d.linear_beta, d.routed_scaling_factor, d.eps = 1.0, 0.5, 2.5, 1e-6
        for n in ("w_router", "w_down", "w1", "w2", "w_s1", "w_s2", "w_up", "logits", "topk_ids", "topk_weights",
                  "expert_counts", "expert_offsets", "tile_offsets", "row_to_pair", "tile_expert", "pair_to_row",
                  "perm_ws", "latent", "act", "z", "fc2_ws", "shared_act", "shared_out", "norm", "out"):
            setattr(d, n, P)
        d.rows_cap = B.lmoe_permute_rows_cap(8, 896, 16, 16)
        d.perm_ws_bytes = 1 << 20
        d.fc2_ws_bytes = B.lmoe_fc2_workspace_bytes(8, 16, 2048)
        d.shared_stream, d.fold_shared_fc2 = 1, -1
        for k, v in over.items():
            setattr(d, k, v)
        return d

    def create(d):
        h = ctypes.c_void_p()
        st = L.lmoe_layer_create(ctypes.byref(d), ctypes.byref(h))
        assert h.value is None
        return st

    assert L.lmoe_layer_create(None, None) == B.LMOE_ERR_INVALID_ARG
    assert create(desc(H=0)) == B.LMOE_ERR_INVALID_ARG
    assert create(desc(dtype=B.LMOE_MXFP8_E4M3)) == B.LMOE_ERR_INVALID_ARG
    assert create(desc(routing=7)) == B.LMOE_ERR_INVALID_ARG
    assert create(desc(w1=None)) == B.LMOE_ERR_INVALID_ARG
    assert create(desc(out=None)) == B.LMOE_ERR_INVALID_ARG
    assert create(desc(mx_experts=1)) == B.LMOE_ERR_INVALID_ARG            # no scales
    assert create(desc(shared_out=None)) == B.LMOE_ERR_INVALID_ARG         # T = 8: the shared FC2 is not folded
    assert create(desc(side_waves=-1)) == B.LMOE_ERR_INVALID_ARG
    assert create(desc(rows_cap=16)) == B.LMOE_ERR_WORKSPACE
    assert create(desc(fc2_ws_bytes=16)) == B.LMOE_ERR_WORKSPACE
    assert create(desc(E=2048, rows_cap=B.lmoe_permute_rows_cap(8, 2048, 16, 16))) == B.LMOE_ERR_UNSUPPORTED
    assert create(desc(K=65, rows_cap=B.lmoe_permute_rows_cap(8, 896, 65, 16),
                       fc2_ws_bytes=B.lmoe_fc2_workspace_bytes(8, 65, 2048))) == B.LMOE_ERR_INVALID_ARG  # K <= 64
    assert create(desc(H=7160)) == B.LMOE_ERR_UNSUPPORTED                   # projections: H % 128
    assert create(desc(routing=B.LMOE_ROUTE_GROUPED, n_group=3)) == B.LMOE_ERR_INVALID_ARG   # E % n_group
    assert create(desc(beta=0.0)) == B.LMOE_ERR_INVALID_ARG


def test_product_path_refuses_to_run_without_the_library(monkeypatch):
    from latent_moe_layer_sigmoid_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", os.path.join(ROOT, "_build", "does_not_exist.so"))
    with pytest.raises(RuntimeError):
        binding.lib()
