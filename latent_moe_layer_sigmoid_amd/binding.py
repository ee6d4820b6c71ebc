"""ctypes binding of liblmoe.so: the C ABI declared in include/lmoe.h, one Python
function per entry point with the same name and argument order.

Marshalling only: tensors are passed as device pointers (None = NULL), the stream
defaults to torch's current stream, and a non-OK status raises LmoeError. Every step
of the layer runs in the library's HIP kernels; nothing here computes.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblmoe.so")

LMOE_OK, LMOE_ERR_INVALID_ARG, LMOE_ERR_UNSUPPORTED, LMOE_ERR_WORKSPACE, LMOE_ERR_HIP = range(5)
LMOE_F32, LMOE_BF16, LMOE_MXFP8_E4M3, LMOE_MXFP4_E2M1 = range(4)

STATUS_NAMES = {0: "LMOE_OK", 1: "LMOE_ERR_INVALID_ARG", 2: "LMOE_ERR_UNSUPPORTED",
                3: "LMOE_ERR_WORKSPACE", 4: "LMOE_ERR_HIP"}


class LmoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {STATUS_NAMES.get(status, status)}")


_i, _f, _p, _z = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

# (name, restype, argtypes) exactly as declared in include/lmoe.h
SIGNATURES = [
    ("lmoe_abi_version", _i, []),
    ("lmoe_status_string", ctypes.c_char_p, [_i]),
    ("lmoe_pack_weights", _i, [_i, _i, _i, _i, _p, _p, _p]),
    ("lmoe_pack_mxfp4_weights", _i, [_i, _i, _i, _p, _p, _p, _p, _p]),
    ("lmoe_linear", _i, [_i, _i, _i, _i, _p, _i, _p, _i, _p, _p]),
    ("lmoe_linear_multi", _i, [_i, _i, _i, _p, _i, _p, _p, _p, _p, _p, _f, _f, _p]),
    ("lmoe_linear_multi_workspace_bytes", _z, [_i, _i, _i, _i, _p, _p]),
    ("lmoe_linear_multi_ws", _i, [_i, _i, _i, _p, _i, _p, _p, _p, _p, _p, _f, _f, _p, _z, _p]),
    ("lmoe_route", _i, [_i, _i, _i, _p, _p, _f, _i, _p, _p, _p]),
    ("lmoe_route_grouped", _i, [_i, _i, _i, _i, _i, _p, _p, _f, _i, _p, _p, _p]),
    ("lmoe_route_renormalize", _i, [_i, _i, _i, _p, _p, _p, _p]),
    ("lmoe_permute_workspace_bytes", _z, [_i, _i, _i]),
    ("lmoe_permute_rows_cap", _i, [_i, _i, _i, _i]),
    ("lmoe_permute", _i, [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _i, _p, _z, _p]),
    ("lmoe_permute_noalloc_max_bytes", _z, []),
    ("lmoe_permute_noalloc", _i, [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _i, _p]),
    ("lmoe_route_permute", _i, [_i, _i, _i, _p, _p, _f, _i, _p, _p, _i, _p, _p, _p, _p, _p, _p, _i, _p, _z, _p]),
    ("lmoe_quant_mxfp8", _i, [_i, _i, _i, _p, _p, _p, _p]),
    ("lmoe_fc1_situ", _i, [_i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _i, _p, _p, _f, _f, _i, _p, _p, _i,
                           _p]),
    ("lmoe_fc1_situ_capped", _i, [_i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _i, _p, _p, _f, _f, _i, _p, _p,
                                  _i, _i, _p]),
    ("lmoe_fc2_workspace_bytes", _z, [_i, _i, _i]),
    ("lmoe_fc2_combine", _i, [_i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _i, _p, _p, _p, _i, _p, _i, _p,
                              _z, _p]),
    ("lmoe_fc2_combine_norm", _i, [_i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _i, _p, _p, _p, _p, _i, _p, _z, _p, _f,
                                   _i, _p, _p]),
    ("lmoe_tail", _i, [_i, _i, _i, _p, _p, _f, _p, _p, _i, _p, _p, _p]),
    ("lmoe_tail_shared", _i, [_i, _i, _i, _i, _p, _p, _f, _p, _p, _p, _i, _p, _p, _p]),
    ("lmoe_tail_shared_workspace_bytes", _z, [_i, _i, _i, _i, _i]),
    ("lmoe_tail_shared_ws", _i, [_i, _i, _i, _i, _p, _p, _f, _p, _p, _p, _i, _p, _p, _p, _z, _p]),
    ("lmoe_situ_masked", _i, [_i, _i, _i, _i, _p, _p, _f, _f, _p, _p]),
    ("lmoe_layer_desc_bytes", _z, []),
    ("lmoe_layer_create", _i, [_p, _p]),
    ("lmoe_layer_forward", _i, [_p, _p, _p]),
    ("lmoe_layer_capture", _i, [_p, _p, _p]),
    ("lmoe_layer_replay", _i, [_p, _p]),
    ("lmoe_layer_destroy", None, [_p]),
]

LMOE_ROUTE_SIGMOID, LMOE_ROUTE_GROUPED, LMOE_ROUTE_RENORMALIZE = range(3)


class LayerDesc(ctypes.Structure):
    """lmoe_layer_desc of include/lmoe.h, field for field."""
    _fields_ = (
        [(n, _i) for n in ("T", "H", "L", "E", "K", "d", "I", "tile_m", "dtype", "mx_experts", "routing", "n_group",
                           "topk_group")]
        + [(n, _f) for n in ("beta", "linear_beta", "routed_scaling_factor", "eps")]
        + [(n, _p) for n in ("w_router", "bias", "w_down", "w1", "w1_scales", "w2", "w2_scales", "w_s1", "w_s2",
                             "gamma", "w_up", "logits", "topk_ids", "topk_weights", "expert_counts",
                             "expert_offsets", "tile_offsets", "row_to_pair", "tile_expert", "pair_to_row")]
        + [("rows_cap", _i), ("perm_ws", _p), ("perm_ws_bytes", _z)]
        + [(n, _p) for n in ("latent", "latent_q", "latent_scales", "act", "act_scales", "z", "fc2_ws")]
        + [("fc2_ws_bytes", _z)]
        + [(n, _p) for n in ("shared_act", "shared_out", "norm", "out", "front_ws")]
        + [("front_ws_bytes", _z), ("tail_ws", _p), ("tail_ws_bytes", _z)]
        + [(n, _i) for n in ("shared_stream", "fold_shared_fc2", "side_waves")]
        + [("side_stream", _p)]
    )

_lib = None


def lib():
    """Load liblmoe.so (built in-tree by build_lib); fails loudly when it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m latent_moe_layer_sigmoid_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a tensor, int or None, got {type(t)}")
    if not t.is_cuda:
        raise ValueError("tensor arguments must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    return int(s)


def _check(fn, st):
    if st != LMOE_OK:
        raise LmoeError(fn, st)


def lmoe_abi_version():
    return lib().lmoe_abi_version()


def lmoe_status_string(status):
    return lib().lmoe_status_string(status).decode()


def lmoe_pack_weights(batch, N, Kd, dtype, src, dst, stream=None):
    _check("lmoe_pack_weights", lib().lmoe_pack_weights(batch, N, Kd, dtype, _ptr(src), _ptr(dst), _stream(stream)))


def packed(w, dtype=None, stream=None):
    """A packed copy of weight tensor w ([N, Kd] or [batch, N, Kd], F32 or BF16)."""
    if dtype is None:
        dtype = LMOE_F32 if w.dtype == torch.float32 else LMOE_BF16
    batch = w.shape[0] if w.dim() == 3 else 1
    out = torch.empty_like(w)
    lmoe_pack_weights(batch, w.shape[-2], w.shape[-1], dtype, w, out, stream)
    return out


def lmoe_linear(M, N, Kd, x_dtype, x, w_dtype, w, y_dtype, y, stream=None):
    _check("lmoe_linear", lib().lmoe_linear(M, N, Kd, x_dtype, _ptr(x), w_dtype, _ptr(w), y_dtype, _ptr(y),
                                            _stream(stream)))


def lmoe_pack_mxfp4_weights(batch, N, Kd, codes_src, scales_src, codes_dst, scales_dst, stream=None):
    _check("lmoe_pack_mxfp4_weights", lib().lmoe_pack_mxfp4_weights(batch, N, Kd, _ptr(codes_src), _ptr(scales_src),
                                                                    _ptr(codes_dst), _ptr(scales_dst),
                                                                    _stream(stream)))


def packed_mxfp4(codes, scales, stream=None):
    """Packed copies of MXFP4 weights: codes [(batch,) N, Kd/2] and scales [(batch,) N, Kd/32]."""
    batch = codes.shape[0] if codes.dim() == 3 else 1
    N, Kd = codes.shape[-2], codes.shape[-1] * 2
    c, s = torch.empty_like(codes), torch.empty_like(scales)
    lmoe_pack_mxfp4_weights(batch, N, Kd, codes, scales, c, s, stream)
    return c, s


def lmoe_linear_multi(M, Kd, x_dtype, x, n_proj, N, w, y_dtype, y, situ, beta, linear_beta, stream=None):
    """N, w, y_dtype, y, situ: sequences of length n_proj (situ may be None)."""
    n = int(n_proj)
    Na = (ctypes.c_int * n)(*N)
    wa = (ctypes.c_void_p * n)(*[_ptr(t) for t in w])
    ta = (ctypes.c_int * n)(*y_dtype)
    ya = (ctypes.c_void_p * n)(*[_ptr(t) for t in y])
    sa = None if situ is None else (ctypes.c_int * n)(*[int(v) for v in situ])
    _check("lmoe_linear_multi", lib().lmoe_linear_multi(M, Kd, x_dtype, _ptr(x), n, Na, wa, ta, ya, sa,
                                                        float(beta), float(linear_beta), _stream(stream)))


def lmoe_linear_multi_workspace_bytes(M, Kd, x_dtype, n_proj, N, situ=None):
    n = int(n_proj)
    Na = (ctypes.c_int * n)(*N)
    sa = None if situ is None else (ctypes.c_int * n)(*[int(v) for v in situ])
    return int(lib().lmoe_linear_multi_workspace_bytes(M, Kd, x_dtype, n, Na, sa))


def lmoe_linear_multi_ws(M, Kd, x_dtype, x, n_proj, N, w, y_dtype, y, situ, beta, linear_beta, workspace,
                         workspace_bytes, stream=None):
    n = int(n_proj)
    Na = (ctypes.c_int * n)(*N)
    wa = (ctypes.c_void_p * n)(*[_ptr(t) for t in w])
    ta = (ctypes.c_int * n)(*y_dtype)
    ya = (ctypes.c_void_p * n)(*[_ptr(t) for t in y])
    sa = None if situ is None else (ctypes.c_int * n)(*[int(v) for v in situ])
    _check("lmoe_linear_multi_ws", lib().lmoe_linear_multi_ws(M, Kd, x_dtype, _ptr(x), n, Na, wa, ta, ya, sa,
                                                              float(beta), float(linear_beta), _ptr(workspace),
                                                              int(workspace_bytes), _stream(stream)))


def lmoe_route(T, E, K, logits, bias, routed_scaling_factor, renormalize, topk_ids, topk_weights, stream=None):
    _check("lmoe_route", lib().lmoe_route(T, E, K, _ptr(logits), _ptr(bias), float(routed_scaling_factor),
                                          int(renormalize), _ptr(topk_ids), _ptr(topk_weights), _stream(stream)))


def lmoe_route_grouped(T, E, K, n_group, topk_group, logits, bias, routed_scaling_factor, renormalize, topk_ids,
                       topk_weights, stream=None):
    _check("lmoe_route_grouped", lib().lmoe_route_grouped(T, E, K, n_group, topk_group, _ptr(logits), _ptr(bias),
                                                          float(routed_scaling_factor), int(renormalize),
                                                          _ptr(topk_ids), _ptr(topk_weights), _stream(stream)))


def lmoe_route_renormalize(T, E, K, logits, topk_ids, topk_weights, stream=None):
    _check("lmoe_route_renormalize", lib().lmoe_route_renormalize(T, E, K, _ptr(logits), _ptr(topk_ids),
                                                                  _ptr(topk_weights), _stream(stream)))


def lmoe_permute_workspace_bytes(T, E, K):
    return int(lib().lmoe_permute_workspace_bytes(T, E, K))


def lmoe_permute_rows_cap(T, E, K, tile_m):
    return int(lib().lmoe_permute_rows_cap(T, E, K, tile_m))


def lmoe_permute(T, E, K, tile_m, topk_ids, expert_counts, expert_offsets, tile_offsets, row_to_pair,
                 tile_expert, pair_to_row, rows_cap, workspace, workspace_bytes, stream=None):
    _check("lmoe_permute", lib().lmoe_permute(T, E, K, tile_m, _ptr(topk_ids), _ptr(expert_counts),
                                              _ptr(expert_offsets), _ptr(tile_offsets), _ptr(row_to_pair),
                                              _ptr(tile_expert), _ptr(pair_to_row), rows_cap, _ptr(workspace),
                                              int(workspace_bytes), _stream(stream)))


def lmoe_permute_noalloc_max_bytes():
    return int(lib().lmoe_permute_noalloc_max_bytes())


def lmoe_permute_noalloc(T, E, K, tile_m, topk_ids, expert_counts, expert_offsets, tile_offsets, row_to_pair,
                         tile_expert, pair_to_row, rows_cap, stream=None):
    _check("lmoe_permute_noalloc", lib().lmoe_permute_noalloc(T, E, K, tile_m, _ptr(topk_ids), _ptr(expert_counts),
                                                              _ptr(expert_offsets), _ptr(tile_offsets),
                                                              _ptr(row_to_pair), _ptr(tile_expert), _ptr(pair_to_row),
                                                              rows_cap, _stream(stream)))


def lmoe_route_permute(T, E, K, logits, bias, routed_scaling_factor, renormalize, topk_ids, topk_weights, tile_m,
                       expert_counts, expert_offsets, tile_offsets, row_to_pair, tile_expert, pair_to_row, rows_cap,
                       workspace, workspace_bytes, stream=None):
    _check("lmoe_route_permute", lib().lmoe_route_permute(
        T, E, K, _ptr(logits), _ptr(bias), float(routed_scaling_factor), int(renormalize), _ptr(topk_ids),
        _ptr(topk_weights), tile_m, _ptr(expert_counts), _ptr(expert_offsets), _ptr(tile_offsets), _ptr(row_to_pair),
        _ptr(tile_expert), _ptr(pair_to_row), rows_cap, _ptr(workspace), int(workspace_bytes), _stream(stream)))


def lmoe_quant_mxfp8(rows, cols, in_dtype, inp, codes, scales, stream=None):
    _check("lmoe_quant_mxfp8", lib().lmoe_quant_mxfp8(rows, cols, in_dtype, _ptr(inp), _ptr(codes), _ptr(scales),
                                                      _stream(stream)))


def lmoe_fc1_situ(T, E, K, in_dim, d, tile_m, a_dtype, a, a_scale, row_to_pair, tile_expert, w_dtype, w1,
                  w1_scale, beta, linear_beta, act_dtype, act, act_scale, rows_cap, stream=None):
    _check("lmoe_fc1_situ", lib().lmoe_fc1_situ(T, E, K, in_dim, d, tile_m, a_dtype, _ptr(a), _ptr(a_scale),
                                                _ptr(row_to_pair), _ptr(tile_expert), w_dtype, _ptr(w1),
                                                _ptr(w1_scale), float(beta), float(linear_beta), act_dtype,
                                                _ptr(act), _ptr(act_scale), rows_cap, _stream(stream)))


def lmoe_fc1_situ_capped(T, E, K, in_dim, d, tile_m, a_dtype, a, a_scale, row_to_pair, tile_expert, w_dtype, w1,
                         w1_scale, beta, linear_beta, act_dtype, act, act_scale, rows_cap, max_waves, stream=None):
    _check("lmoe_fc1_situ_capped",
           lib().lmoe_fc1_situ_capped(T, E, K, in_dim, d, tile_m, a_dtype, _ptr(a), _ptr(a_scale), _ptr(row_to_pair),
                                      _ptr(tile_expert), w_dtype, _ptr(w1), _ptr(w1_scale), float(beta),
                                      float(linear_beta), act_dtype, _ptr(act), _ptr(act_scale), rows_cap,
                                      max_waves, _stream(stream)))


def lmoe_fc2_workspace_bytes(T, K, out_dim):
    return int(lib().lmoe_fc2_workspace_bytes(T, K, out_dim))


def lmoe_fc2_combine(T, E, K, d, out_dim, tile_m, act_dtype, act, act_scale, row_to_pair, tile_expert, w_dtype,
                     w2, w2_scale, topk_weights, out_dtype, out, rows_cap, workspace, workspace_bytes, stream=None):
    _check("lmoe_fc2_combine", lib().lmoe_fc2_combine(T, E, K, d, out_dim, tile_m, act_dtype, _ptr(act),
                                                      _ptr(act_scale), _ptr(row_to_pair), _ptr(tile_expert),
                                                      w_dtype, _ptr(w2), _ptr(w2_scale), _ptr(topk_weights),
                                                      out_dtype, _ptr(out), rows_cap, _ptr(workspace),
                                                      int(workspace_bytes), _stream(stream)))


def lmoe_fc2_combine_norm(T, E, K, d, out_dim, tile_m, act_dtype, act, act_scale, row_to_pair, tile_expert, w_dtype,
                          w2, w2_scale, topk_weights, z, rows_cap, workspace, workspace_bytes, gamma, eps, norm_dtype,
                          norm_out, stream=None):
    _check("lmoe_fc2_combine_norm", lib().lmoe_fc2_combine_norm(
        T, E, K, d, out_dim, tile_m, act_dtype, _ptr(act), _ptr(act_scale), _ptr(row_to_pair), _ptr(tile_expert),
        w_dtype, _ptr(w2), _ptr(w2_scale), _ptr(topk_weights), _ptr(z), rows_cap, _ptr(workspace),
        int(workspace_bytes), _ptr(gamma), float(eps), norm_dtype, _ptr(norm_out), _stream(stream)))


def lmoe_tail(T, L, H, latent, gamma, eps, w_up, shared, io_dtype, out, norm_out, stream=None):
    _check("lmoe_tail", lib().lmoe_tail(T, L, H, _ptr(latent), _ptr(gamma), float(eps), _ptr(w_up), _ptr(shared),
                                        io_dtype, _ptr(out), _ptr(norm_out), _stream(stream)))


def lmoe_tail_shared(T, L, H, I, latent, gamma, eps, w_up, shared_act, w_s2, io_dtype, out, norm_out, stream=None):
    _check("lmoe_tail_shared", lib().lmoe_tail_shared(T, L, H, I, _ptr(latent), _ptr(gamma), float(eps), _ptr(w_up),
                                                      _ptr(shared_act), _ptr(w_s2), io_dtype, _ptr(out),
                                                      _ptr(norm_out), _stream(stream)))


def lmoe_tail_shared_workspace_bytes(T, L, H, I, io_dtype):
    return int(lib().lmoe_tail_shared_workspace_bytes(T, L, H, I, io_dtype))


def lmoe_tail_shared_ws(T, L, H, I, latent, gamma, eps, w_up, shared_act, w_s2, io_dtype, out, norm_out, workspace,
                        workspace_bytes, stream=None):
    _check("lmoe_tail_shared_ws", lib().lmoe_tail_shared_ws(T, L, H, I, _ptr(latent), _ptr(gamma), float(eps),
                                                            _ptr(w_up), _ptr(shared_act), _ptr(w_s2), io_dtype,
                                                            _ptr(out), _ptr(norm_out), _ptr(workspace),
                                                            int(workspace_bytes), _stream(stream)))


def lmoe_situ_masked(E, T_max, d, dtype, inp, expert_num_tokens, beta, linear_beta, out, stream=None):
    _check("lmoe_situ_masked", lib().lmoe_situ_masked(E, T_max, d, dtype, _ptr(inp), _ptr(expert_num_tokens),
                                                      float(beta), float(linear_beta), _ptr(out), _stream(stream)))


def lmoe_layer_desc_bytes():
    return lib().lmoe_layer_desc_bytes()


def lmoe_layer_create(desc):
    """A layer object for `desc` (a LayerDesc); returns its handle (an int)."""
    if ctypes.sizeof(LayerDesc) != lib().lmoe_layer_desc_bytes():
        raise RuntimeError("LayerDesc does not match the library's lmoe_layer_desc")
    h = ctypes.c_void_p()
    _check("lmoe_layer_create", lib().lmoe_layer_create(ctypes.byref(desc), ctypes.byref(h)))
    return h.value


def lmoe_layer_forward(layer, x, stream=None):
    _check("lmoe_layer_forward", lib().lmoe_layer_forward(layer, _ptr(x), _stream(stream)))


def lmoe_layer_capture(layer, x, stream=None):
    _check("lmoe_layer_capture", lib().lmoe_layer_capture(layer, _ptr(x), _stream(stream)))


def lmoe_layer_replay(layer, stream=None):
    _check("lmoe_layer_replay", lib().lmoe_layer_replay(layer, _stream(stream)))


def lmoe_layer_destroy(layer):
    lib().lmoe_layer_destroy(layer)
