"""One latent-MoE layer forward composed from the C ABI (TensorRT-LLM PR 20541,
"Description": router GEMM, latent down projection, input quantization, routing, FC1 /
FC2, then the routed reduction with RMSNorm and the latent up projection; vLLM PR 50088,
commit 7 and the vLLM latent_moe_runner API page for the latent tail).

This module only sequences library calls and owns device buffers (allocated with torch
once per token count); every step runs in liblmoe's HIP kernels.
"""
import weakref
from dataclasses import dataclass

import torch

from . import binding as B


@dataclass
class LayerShape:
    H: int
    L: int
    E: int
    K: int
    d: int
    I: int
    dtype: str            # "f32" or "bf16"
    experts: str          # "dense" or "mx"
    beta: float
    linear_beta: float
    rsf: float
    eps: float
    tile_m: int = 16
    routing: str = "sigmoid"   # "sigmoid" (bias-corrected, DeepSeekV3) or "renormalize"
    n_group: int = 1          # grouped top-k for sigmoid routing
    topk_group: int = 1


# The extra streams of the layer, one of each kind per device, shared by every layer of the
# process: HIP gives a process a few hardware queues (four by default) and spreads its
# streams over them, so every new stream risks landing on the main stream's queue, where
# its work would run after the main stream's instead of beside it (measured: an MX step
# 0.59 -> 0.73 ms with a freshly created side stream in a process holding several). Layers
# run one after another, so sharing costs no overlap.
_AUX_STREAMS = {}


def _aux_stream(device, kind):
    key = (str(device), kind)
    if key not in _AUX_STREAMS:
        _AUX_STREAMS[key] = torch.cuda.Stream(device)   # default priority
    return _AUX_STREAMS[key]


def _lmoe_dtype(dtype):
    return B.LMOE_F32 if dtype == "f32" else B.LMOE_BF16


def _torch_dtype(dtype):
    return torch.float32 if dtype == "f32" else torch.bfloat16


class LatentMoELayer:
    """Holds device weights and runs the layer through liblmoe.

    weights: dict of row-major device tensors W_r [E,H], bias [E] fp32, W_down [L,H],
    W1 [E,2d,L] / W2 [E,L,d] (or W1_codes/W1_scales/W2_codes/W2_scales for MX experts),
    W_s1 [2I,H], W_s2 [H,I], gamma [L], W_up [H,L]; the projections are packed on the
    device (lmoe_pack_weights) when the layer is built."""

    def __init__(self, shape: LayerShape, weights: dict, device="cuda", fused=True, shared_stream=False,
                 router_stream=False, fold_shared_fc2=None, side_waves=512):
        B.lib()   # fail loudly now if the library is missing
        self.s = shape
        # fused: the hidden-input projections share one launch (lmoe_linear_multi) and the
        # shared expert's FC2 is folded into the up projection (lmoe_tail_shared);
        # otherwise every step is its own call.
        self.fused = fused
        # shared_stream: the shared expert runs on a second stream, concurrently with the
        # router GEMM, routing, permutation and the routed experts, and the tail waits for
        # it (TensorRT-LLM PR 20541, "Commit 2": shared experts on their own stream, joined
        # by an event before the routed reduction). Same kernels; the side stream's narrower
        # shared FC1 (side_waves) sums K in another order, so the shared output can differ
        # from the one-stream schedule's in the last bf16 bit.
        self.shared_stream = shared_stream or router_stream
        # router_stream: additionally, the router GEMM, routing and permutation run on a
        # router stream while the main stream computes the latent down projection
        # (TensorRT-LLM PR 20541, "Commit 2": router stream, shared stream, main stream).
        self.router_stream = router_stream
        # fold_shared_fc2 (with a second stream): the side stream runs only the shared FC1
        # and the tail computes the shared FC2 and the up projection in one call
        # (lmoe_tail_shared); None: fold when the token count takes the tiled GEMMs
        self.fold_shared_fc2 = fold_shared_fc2
        # side_waves: wavefronts the side stream's shared FC1 aims for when it streams its
        # weights (lmoe_fc1_situ_capped; 0: the library default of 2048). A narrower launch
        # leaves more of the HBM bandwidth to the main stream's router GEMM and experts,
        # while the shared expert still finishes before the tail needs it.
        self.side_waves = side_waves
        self.device = torch.device(device)
        # extra streams at the default priority
        self._side = _aux_stream(self.device, "side") if self.shared_stream else None
        self._router = _aux_stream(self.device, "router") if router_stream else None
        self._bufs = {}
        # weights go to HBM in the packed MFMA-operand layout once, at construction
        self.w = {}
        for k, v in weights.items():
            if k in ("W_r", "W_down", "W1", "W2", "W_s1", "W_s2", "W_up"):
                self.w[k] = B.packed(v)
            elif k in ("W1_codes", "W2_codes"):
                name = k[:2]
                self.w[k], self.w[name + "_scales"] = B.packed_mxfp4(v, weights[name + "_scales"])
            elif k not in ("W1_scales", "W2_scales"):
                self.w[k] = v
        torch.cuda.synchronize(self.device)

    def reshaped(self, **changes):
        """A layer over the same packed device weights with some LayerShape fields changed
        (e.g. tile_m for another batch size regime), its own buffers and streams."""
        import copy
        import dataclasses
        other = copy.copy(self)
        other.s = dataclasses.replace(self.s, **changes)
        other._bufs = {}
        other._side = self._side
        other._router = self._router
        return other

    def buffers(self, T):
        if T in self._bufs:
            return self._bufs[T]
        s, dev = self.s, self.device
        dt = _torch_dtype(s.dtype)
        rows_cap = B.lmoe_permute_rows_cap(T, s.E, s.K, s.tile_m)
        pw = B.lmoe_permute_workspace_bytes(T, s.E, s.K)
        fw = B.lmoe_fc2_workspace_bytes(T, s.K, s.L)
        i32 = dict(dtype=torch.int32, device=dev)
        b = dict(
            rows_cap=rows_cap,
            logits=torch.empty(T, s.E, dtype=torch.float32, device=dev),
            ids=torch.empty(T, s.K, **i32),
            weights=torch.empty(T, s.K, dtype=torch.float32, device=dev),
            counts=torch.empty(s.E, **i32),
            offsets=torch.empty(s.E + 1, **i32),
            tile_offsets=torch.empty(s.E + 1, **i32),
            row_to_pair=torch.empty(max(rows_cap, 1), **i32),
            tile_expert=torch.empty(max(rows_cap // s.tile_m, 1), **i32),
            pair_to_row=torch.empty(max(T * s.K, 1), **i32),
            perm_ws=torch.empty(max(pw, 1), dtype=torch.uint8, device=dev),
            perm_ws_bytes=pw,
            x=torch.empty(T, s.L, dtype=dt, device=dev),
            z=torch.empty(T, s.L, dtype=torch.float32, device=dev),
            fc2_ws=torch.empty(max(fw // 4, 1), dtype=torch.float32, device=dev),
            fc2_ws_bytes=fw,
            act_s=torch.empty(T, s.I, dtype=dt, device=dev),
            sh=torch.empty(T, s.H, dtype=dt, device=dev),
            n=torch.empty(T, s.L, dtype=dt, device=dev),
            out=torch.empty(T, s.H, dtype=dt, device=dev),
        )
        # split-K workspace of the front projections (used when their tiles alone would
        # leave CUs idle): the two- and three-projection variants
        dtl = _lmoe_dtype(s.dtype)
        fw2 = B.lmoe_linear_multi_workspace_bytes(T, s.H, dtl, 2, [s.E, s.L], None)
        fw3 = B.lmoe_linear_multi_workspace_bytes(T, s.H, dtl, 3, [s.E, s.L, s.I], [0, 0, 1])
        fws = max(fw2, fw3)
        b["front_ws"] = torch.empty(max(fws // 4, 1), dtype=torch.float32, device=dev) if fws else None
        b["front_ws_bytes"] = fws
        # split-K workspace of the fused tail (shared FC2 + up projection)
        tws = B.lmoe_tail_shared_workspace_bytes(T, s.L, s.H, s.I, dtl)
        b["tail_ws"] = torch.empty(max(tws // 4, 1), dtype=torch.float32, device=dev) if tws else None
        b["tail_ws_bytes"] = tws
        if s.experts == "mx":
            b["xq"] = torch.empty(T, s.L, dtype=torch.uint8, device=dev)
            b["xs"] = torch.empty(T, s.L // 32, dtype=torch.uint8, device=dev)
            b["act"] = torch.empty(max(rows_cap, 1), s.d, dtype=torch.uint8, device=dev)
            b["act_scale"] = torch.empty(max(rows_cap, 1), s.d // 32, dtype=torch.uint8, device=dev)
        else:
            b["act"] = torch.empty(max(rows_cap, 1), s.d, dtype=dt, device=dev)
            b["act_scale"] = None
        self._bufs[T] = b
        return b

    def forward(self, X, stream=None, timer=None):
        """Run the layer on X [T, H]; returns the output buffer [T, H] (overwritten by the
        next call with the same T). Intermediates stay in self.buffers(T).

        timer: optional StepTimer; it records HIP events on the launch stream between the
        library calls (one pair per step of the layer)."""
        s, w = self.s, self.w
        T = X.shape[0]
        b = self.buffers(T)
        dt = _lmoe_dtype(s.dtype)
        mark = timer.mark if timer is not None else (lambda name: None)
        if self.shared_stream:
            return self._forward_two_streams(X, b, stream, mark)
        if self.fused:
            # router GEMM, latent down projection, shared FC1 + SituGLU: one launch
            mark("front")
            B.lmoe_linear_multi_ws(T, s.H, dt, X, 3, [s.E, s.L, s.I], [w["W_r"], w["W_down"], w["W_s1"]],
                                   [B.LMOE_F32, dt, dt], [b["logits"], b["x"], b["act_s"]], [0, 0, 1], s.beta,
                                   s.linear_beta, b["front_ws"], b["front_ws_bytes"], stream)
        else:
            # router GEMM -> fp32 logits, latent down projection
            mark("router")
            B.lmoe_linear(T, s.E, s.H, dt, X, dt, w["W_r"], B.LMOE_F32, b["logits"], stream)
            mark("down")
            B.lmoe_linear(T, s.L, s.H, dt, X, dt, w["W_down"], dt, b["x"], stream)
        # routing, permutation, routed experts (fused: FC2 also leaves the normalized latent)
        self._routed(X, b, stream, mark, norm=self.fused)
        if self.fused:
            # shared expert's FC2 folded into the up projection: one GEMM over both K ranges
            mark("tail")
            B.lmoe_tail_shared_ws(T, s.L, s.H, s.I, None, w["gamma"], s.eps, w["W_up"], b["act_s"], w["W_s2"], dt,
                                  b["out"], b["n"], b["tail_ws"], b["tail_ws_bytes"], stream)
        else:
            # shared expert (dense mode: E = K = 1)
            mark("shared_fc1")
            B.lmoe_fc1_situ(T, 1, 1, s.H, s.I, 16, dt, X, None, None, None, dt, w["W_s1"], None, s.beta,
                            s.linear_beta, dt, b["act_s"], None, T, stream)
            mark("shared_fc2")
            B.lmoe_fc2_combine(T, 1, 1, s.I, s.H, 16, dt, b["act_s"], None, None, None, dt, w["W_s2"], None, None,
                               dt, b["sh"], T, None, 0, stream)
            # latent RMSNorm, up projection with the shared add in its epilogue
            mark("tail")
            B.lmoe_tail(T, s.L, s.H, b["z"], w["gamma"], s.eps, w["W_up"], b["sh"], dt, b["out"], b["n"], stream)
        mark(None)
        return b["out"]

    def folds_shared_fc2(self, T):
        """True when a forward pass over T tokens with the shared-expert stream computes the
        shared FC2 inside the tail (the shared output b["sh"] is then not written)."""
        if not self.shared_stream:
            return False
        if self.fold_shared_fc2 is not None:
            return self.fold_shared_fc2
        return T >= 256 and self.s.dtype == "bf16"

    def native(self, T):
        """This layer's step over T tokens as one library object (lmoe_layer_create): the
        same launches as forward() with its schedule, run by lmoe_layer_forward, and
        recordable as a HIP graph inside the library (lmoe_layer_capture / _replay). It
        uses this layer's packed weights and buffers(T). The fused schedules only (one
        stream, or the shared-expert stream without the router stream)."""
        return NativeLayer(self, T)

    def capture(self, X):
        """A HIP graph of one forward pass on the static input X (same buffers as
        forward(X)); graph.replay() reruns the whole layer, reading X's current contents.
        The library records no memset and allocates nothing, so every launch is a kernel
        node; the shared-expert stream, if used, is forked and joined inside the graph."""
        cur = torch.cuda.current_stream(self.device)
        warm = torch.cuda.Stream(self.device)
        warm.wait_stream(cur)
        with torch.cuda.stream(warm):
            self.forward(X)               # buffers exist before capture
        cur.wait_stream(warm)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.forward(X)
        return graph

    def _routed(self, X, b, stream, mark, norm=False):
        """Routing, permutation and the routed experts on `stream`; with norm, the FC2 call
        also leaves the RMS-normalized latent in b["n"] (combine and RMSNorm in one kernel)."""
        T = X.shape[0]
        mark("route_permute")
        self._route(T, b, stream)
        self._experts(T, b, stream, mark, norm)

    def _route(self, T, b, stream):
        """Routing and the permutation on `stream`."""
        s, w = self.s, self.w
        rc = b["rows_cap"]
        if s.routing == "sigmoid" and s.n_group == 1:
            B.lmoe_route_permute(T, s.E, s.K, b["logits"], w["bias"], s.rsf, 1, b["ids"], b["weights"], s.tile_m,
                                 b["counts"], b["offsets"], b["tile_offsets"], b["row_to_pair"], b["tile_expert"],
                                 b["pair_to_row"], rc, b["perm_ws"], b["perm_ws_bytes"], stream)
        else:
            if s.routing == "renormalize":
                B.lmoe_route_renormalize(T, s.E, s.K, b["logits"], b["ids"], b["weights"], stream)
            else:
                B.lmoe_route_grouped(T, s.E, s.K, s.n_group, s.topk_group, b["logits"], w["bias"], s.rsf, 1,
                                     b["ids"], b["weights"], stream)
            B.lmoe_permute(T, s.E, s.K, s.tile_m, b["ids"], b["counts"], b["offsets"], b["tile_offsets"],
                           b["row_to_pair"], b["tile_expert"], b["pair_to_row"], rc, b["perm_ws"],
                           b["perm_ws_bytes"], stream)

    def _experts(self, T, b, stream, mark, norm=False):
        """The routed experts (input quantization for MX, FC1 + SituGLU, FC2 + combine, and
        with norm the RMS-normalized latent) on `stream`."""
        s, w = self.s, self.w
        dt = _lmoe_dtype(s.dtype)
        rc = b["rows_cap"]
        if s.experts == "mx":
            mark("quant")
            B.lmoe_quant_mxfp8(T, s.L, dt, b["x"], b["xq"], b["xs"], stream)
            mark("fc1")
            B.lmoe_fc1_situ(T, s.E, s.K, s.L, s.d, s.tile_m, B.LMOE_MXFP8_E4M3, b["xq"], b["xs"], b["row_to_pair"],
                            b["tile_expert"], B.LMOE_MXFP4_E2M1, w["W1_codes"], w["W1_scales"], s.beta,
                            s.linear_beta, B.LMOE_MXFP8_E4M3, b["act"], b["act_scale"], rc, stream)
            a_dt, a, a_s, w2_dt, w2, w2_s = (B.LMOE_MXFP8_E4M3, b["act"], b["act_scale"], B.LMOE_MXFP4_E2M1,
                                             w["W2_codes"], w["W2_scales"])
        else:
            mark("fc1")
            B.lmoe_fc1_situ(T, s.E, s.K, s.L, s.d, s.tile_m, dt, b["x"], None, b["row_to_pair"], b["tile_expert"],
                            dt, w["W1"], None, s.beta, s.linear_beta, dt, b["act"], None, rc, stream)
            a_dt, a, a_s, w2_dt, w2, w2_s = dt, b["act"], None, dt, w["W2"], None
        mark("fc2")
        if norm:
            B.lmoe_fc2_combine_norm(T, s.E, s.K, s.d, s.L, s.tile_m, a_dt, a, a_s, b["row_to_pair"], b["tile_expert"],
                                    w2_dt, w2, w2_s, b["weights"], b["z"], rc, b["fc2_ws"], b["fc2_ws_bytes"],
                                    w["gamma"], s.eps, dt, b["n"], stream)
        else:
            B.lmoe_fc2_combine(T, s.E, s.K, s.d, s.L, s.tile_m, a_dt, a, a_s, b["row_to_pair"], b["tile_expert"],
                               w2_dt, w2, w2_s, b["weights"], B.LMOE_F32, b["z"], rc, b["fc2_ws"], b["fc2_ws_bytes"],
                               stream)

    def _forward_two_streams(self, X, b, stream, mark):
        """Main stream: router GEMM + down projection (one launch), routing, permutation,
        experts, then RMSNorm + up projection with the shared add. Side stream: the shared
        expert (FC1 + SituGLU, FC2), started once the main stream reaches this call and
        joined by an event before the tail; when folded (fold_shared_fc2), the side stream
        runs only the FC1 and the tail computes the shared FC2 and the up projection in one
        call. With the router stream, the router GEMM,
        routing and permutation run there and the main stream computes the down projection
        meanwhile, then waits for the routing before the experts."""
        s, w = self.s, self.w
        T = X.shape[0]
        dt = _lmoe_dtype(s.dtype)
        main = torch.cuda.current_stream(self.device) if stream is None else stream
        side = self._side
        start = torch.cuda.Event()
        start.record(main)
        side.wait_event(start)            # X is ready and the previous call's tail has read sh
        if not torch.cuda.is_current_stream_capturing():
            X.record_stream(side)
        fold = self.folds_shared_fc2(T)
        # When the shared FC1's 128 x 512 tiles alone fill the CUs (one workgroup holds a
        # whole CU), the main stream also waits until the side stream has taken the fork:
        # the shared FC1 then starts first and shares the chip with the router + down
        # projection, instead of with the routed FC1 by a race between the two queues.
        # Same step time (prefill 3.43-3.44 ms either way), a stable split between the
        # launches. With fewer tiles (T = 1024) the extra wait measured slower.
        forked = None
        if (T + 127) // 128 * ((2 * s.I + 511) // 512) >= 256:
            forked = torch.cuda.Event()
            forked.record(side)
        B.lmoe_fc1_situ_capped(T, 1, 1, s.H, s.I, 16, dt, X, None, None, None, dt, w["W_s1"], None, s.beta,
                               s.linear_beta, dt, b["act_s"], None, T, self.side_waves, side)
        if forked is not None:
            main.wait_event(forked)
        if not fold:
            B.lmoe_fc2_combine(T, 1, 1, s.I, s.H, 16, dt, b["act_s"], None, None, None, dt, w["W_s2"], None, None,
                               dt, b["sh"], T, None, 0, side)
        shared_done = torch.cuda.Event()
        shared_done.record(side)
        if self.router_stream:
            rs = self._router
            rs.wait_event(start)
            if not torch.cuda.is_current_stream_capturing():
                X.record_stream(rs)
            B.lmoe_linear(T, s.E, s.H, dt, X, dt, w["W_r"], B.LMOE_F32, b["logits"], rs)
            self._route(T, b, rs)
            routed = torch.cuda.Event()
            routed.record(rs)
            mark("front")
            B.lmoe_linear(T, s.L, s.H, dt, X, dt, w["W_down"], dt, b["x"], main)
            main.wait_event(routed)
            self._experts(T, b, main, mark, norm=True)
        else:
            mark("front")
            B.lmoe_linear_multi_ws(T, s.H, dt, X, 2, [s.E, s.L], [w["W_r"], w["W_down"]], [B.LMOE_F32, dt],
                                   [b["logits"], b["x"]], None, s.beta, s.linear_beta, b["front_ws"],
                                   b["front_ws_bytes"], main)
            self._routed(X, b, main, mark, norm=True)
        main.wait_event(shared_done)
        mark("tail")
        if fold:
            B.lmoe_tail_shared_ws(T, s.L, s.H, s.I, None, w["gamma"], s.eps, w["W_up"], b["act_s"], w["W_s2"], dt,
                                  b["out"], b["n"], b["tail_ws"], b["tail_ws_bytes"], main)
        else:
            B.lmoe_tail(T, s.L, s.H, None, w["gamma"], s.eps, w["W_up"], b["sh"], dt, b["out"], b["n"], main)
        mark(None)
        return b["out"]


class NativeLayer:
    """A lmoe_layer object over a LatentMoELayer's weights and buffers for T tokens.
    forward(X) enqueues one step (output in buffers(T)["out"]); capture(X) records one
    step reading X into a HIP graph inside the library and replay() launches it."""

    def __init__(self, layer, T):
        if not layer.fused or layer.router_stream:
            raise ValueError("the library's layer step runs the fused schedules without the router stream")
        s, w = layer.s, layer.w
        b = layer.buffers(T)
        mx = s.experts == "mx"
        d = B.LayerDesc()
        d.T, d.H, d.L, d.E, d.K, d.d, d.I, d.tile_m = T, s.H, s.L, s.E, s.K, s.d, s.I, s.tile_m
        d.dtype = _lmoe_dtype(s.dtype)
        d.mx_experts = int(mx)
        if s.routing == "renormalize":
            d.routing = B.LMOE_ROUTE_RENORMALIZE
        else:
            d.routing = B.LMOE_ROUTE_GROUPED if s.n_group > 1 else B.LMOE_ROUTE_SIGMOID
        d.n_group, d.topk_group = s.n_group, s.topk_group
        d.beta, d.linear_beta, d.routed_scaling_factor, d.eps = s.beta, s.linear_beta, s.rsf, s.eps
        P = B._ptr
        d.w_router, d.bias, d.w_down = P(w["W_r"]), P(w.get("bias")), P(w["W_down"])
        if mx:
            d.w1, d.w1_scales = P(w["W1_codes"]), P(w["W1_scales"])
            d.w2, d.w2_scales = P(w["W2_codes"]), P(w["W2_scales"])
        else:
            d.w1, d.w2 = P(w["W1"]), P(w["W2"])
        d.w_s1, d.w_s2, d.gamma, d.w_up = P(w["W_s1"]), P(w["W_s2"]), P(w.get("gamma")), P(w["W_up"])
        d.logits, d.topk_ids, d.topk_weights = P(b["logits"]), P(b["ids"]), P(b["weights"])
        d.expert_counts, d.expert_offsets, d.tile_offsets = P(b["counts"]), P(b["offsets"]), P(b["tile_offsets"])
        d.row_to_pair, d.tile_expert, d.pair_to_row = P(b["row_to_pair"]), P(b["tile_expert"]), P(b["pair_to_row"])
        d.rows_cap, d.perm_ws, d.perm_ws_bytes = b["rows_cap"], P(b["perm_ws"]), b["perm_ws_bytes"]
        d.latent = P(b["x"])
        if mx:
            d.latent_q, d.latent_scales, d.act_scales = P(b["xq"]), P(b["xs"]), P(b["act_scale"])
        d.act, d.z, d.fc2_ws, d.fc2_ws_bytes = P(b["act"]), P(b["z"]), P(b["fc2_ws"]), b["fc2_ws_bytes"]
        d.shared_act, d.shared_out, d.norm, d.out = P(b["act_s"]), P(b["sh"]), P(b["n"]), P(b["out"])
        d.front_ws, d.front_ws_bytes = P(b["front_ws"]), b["front_ws_bytes"]
        d.tail_ws, d.tail_ws_bytes = P(b["tail_ws"]), b["tail_ws_bytes"]
        d.shared_stream = int(layer.shared_stream)
        d.fold_shared_fc2 = -1 if layer.fold_shared_fc2 is None else int(bool(layer.fold_shared_fc2))
        d.side_waves = layer.side_waves
        # the Python layer's own second stream: one more stream of the library's would
        # share a hardware queue with the main stream in a process that holds many
        d.side_stream = layer._side.cuda_stream if layer._side is not None else None
        self.T = T
        self.out = b["out"]
        self._keep = (layer, b, w)      # the tensors behind every pointer stay alive
        self.handle = B.lmoe_layer_create(d)
        # released when the object goes away, or at interpreter exit (before the HIP
        # runtime's own teardown)
        self._finalizer = weakref.finalize(self, B.lmoe_layer_destroy, self.handle)

    def forward(self, X, stream=None):
        B.lmoe_layer_forward(self.handle, X, stream)
        return self.out

    def capture(self, X, stream=None):
        B.lmoe_layer_capture(self.handle, X, stream)

    def replay(self, stream=None):
        B.lmoe_layer_replay(self.handle, stream)

    def close(self):
        """Destroy the library object (the caller has waited for its work)."""
        self._finalizer()
        self.handle = None


class StepTimer:
    """HIP events recorded on the launch stream between the layer's library calls;
    durations() gives the mean milliseconds of each step over the recorded calls."""

    def __init__(self, stream=None):
        self.stream = stream
        self.marks = []          # per forward call: list of (name, event)
        self._cur = None

    def mark(self, name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(self.stream if self.stream is not None else torch.cuda.current_stream())
        if self._cur is None:
            self._cur = []
        self._cur.append((name, ev))
        if name is None:
            self.marks.append(self._cur)
            self._cur = None

    def durations(self):
        acc = {}
        for call in self.marks:
            for (name, a), (_, b) in zip(call[:-1], call[1:]):
                acc.setdefault(name, []).append(a.elapsed_time(b))
        return {k: sum(v) / len(v) for k, v in acc.items()}
