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
    for m in re.finditer(r"(?:lmoe_status|size_t|int|const char\s*\*)\s+(lmoe_\w+)\s*\(([^)]*)\)\s*;", src):
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


def test_product_path_refuses_to_run_without_the_library(monkeypatch):
    from latent_moe_layer_sigmoid_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", os.path.join(ROOT, "_build", "does_not_exist.so"))
    with pytest.raises(RuntimeError):
        binding.lib()
