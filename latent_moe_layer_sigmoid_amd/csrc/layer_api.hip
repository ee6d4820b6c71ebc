// One forward step of the layer strung from the C-ABI calls, and its HIP graph (the
// lmoe_layer_* entry points of include/lmoe.h). Host code only: every kernel it runs is
// launched by the calls in lmoe_api.hip.
//
// The schedule is the benchmark's (TensorRT-LLM PR 20541, "Commit 2": the shared experts
// on their own stream, joined by an event before the routed reduction): the main stream
// runs the router GEMM + latent down projection, routing + permutation, the routed FC1 and
// FC2 + combine + RMSNorm, then waits for the shared expert and runs the tail; the layer's
// second stream runs the shared expert. The same PR measures its decode steps under CUDA
// graphs and checks graph runs bitwise against eager ones ("Test Coverage"); here the step
// can be recorded once into a HIP graph inside the library and replayed.
#include <math.h>

#include <new>

#include "lmoe.h"

struct lmoe_layer {
  lmoe_layer_desc d;
  int device;
  hipStream_t side;
  bool own_side;
  hipEvent_t ev_start, ev_fork, ev_shared;
  hipGraphExec_t exec;
};

namespace {

bool dense_dtype(lmoe_dtype t) { return t == LMOE_F32 || t == LMOE_BF16; }

// shared FC2 folded into the tail: asked for, or (-1) by token count as the benchmark does
bool folds(const lmoe_layer_desc& d) {
  if (!d.shared_stream) return true;
  if (d.fold_shared_fc2 >= 0) return d.fold_shared_fc2 != 0;
  return d.T >= 256 && d.dtype == LMOE_BF16;
}

// the shared FC1's 128 x 512 tiles alone fill the CUs: the main stream also waits for the
// side stream's fork, so the shared FC1 starts first (same rule as the Python layer)
bool fork_wait(const lmoe_layer_desc& d) {
  return (long)(d.T + 127) / 128 * ((2L * d.I + 511) / 512) >= 256;
}

lmoe_status hip_ok(hipError_t e) { return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP; }

lmoe_status front(const lmoe_layer_desc& d, const void* X, bool with_shared, hipStream_t s) {
  const int N[3] = {d.E, d.L, d.I};
  const void* w[3] = {d.w_router, d.w_down, d.w_s1};
  const lmoe_dtype yt[3] = {LMOE_F32, d.dtype, d.dtype};
  void* y[3] = {d.logits, d.latent, d.shared_act};
  const int situ[3] = {0, 0, 1};
  return lmoe_linear_multi_ws(d.T, d.H, d.dtype, X, with_shared ? 3 : 2, N, w, yt, y, situ, d.beta, d.linear_beta,
                              d.front_ws, d.front_ws_bytes, s);
}

lmoe_status route(const lmoe_layer_desc& d, hipStream_t s) {
  if (d.routing == LMOE_ROUTE_SIGMOID)
    return lmoe_route_permute(d.T, d.E, d.K, d.logits, d.bias, d.routed_scaling_factor, 1, d.topk_ids,
                              d.topk_weights, d.tile_m, d.expert_counts, d.expert_offsets, d.tile_offsets,
                              d.row_to_pair, d.tile_expert, d.pair_to_row, d.rows_cap, d.perm_ws, d.perm_ws_bytes,
                              s);
  lmoe_status st = d.routing == LMOE_ROUTE_RENORMALIZE
                       ? lmoe_route_renormalize(d.T, d.E, d.K, d.logits, d.topk_ids, d.topk_weights, s)
                       : lmoe_route_grouped(d.T, d.E, d.K, d.n_group, d.topk_group, d.logits, d.bias,
                                            d.routed_scaling_factor, 1, d.topk_ids, d.topk_weights, s);
  if (st != LMOE_OK) return st;
  return lmoe_permute(d.T, d.E, d.K, d.tile_m, d.topk_ids, d.expert_counts, d.expert_offsets, d.tile_offsets,
                      d.row_to_pair, d.tile_expert, d.pair_to_row, d.rows_cap, d.perm_ws, d.perm_ws_bytes, s);
}

lmoe_status experts(const lmoe_layer_desc& d, hipStream_t s) {
  lmoe_status st;
  if (d.mx_experts) {
    st = lmoe_quant_mxfp8(d.T, d.L, d.dtype, d.latent, d.latent_q, d.latent_scales, s);
    if (st != LMOE_OK) return st;
    st = lmoe_fc1_situ(d.T, d.E, d.K, d.L, d.d, d.tile_m, LMOE_MXFP8_E4M3, d.latent_q, d.latent_scales,
                       d.row_to_pair, d.tile_expert, LMOE_MXFP4_E2M1, d.w1, d.w1_scales, d.beta, d.linear_beta,
                       LMOE_MXFP8_E4M3, d.act, d.act_scales, d.rows_cap, s);
  } else {
    st = lmoe_fc1_situ(d.T, d.E, d.K, d.L, d.d, d.tile_m, d.dtype, d.latent, nullptr, d.row_to_pair, d.tile_expert,
                       d.dtype, d.w1, nullptr, d.beta, d.linear_beta, d.dtype, d.act, nullptr, d.rows_cap, s);
  }
  if (st != LMOE_OK) return st;
  const lmoe_dtype at = d.mx_experts ? LMOE_MXFP8_E4M3 : d.dtype;
  const lmoe_dtype wt = d.mx_experts ? LMOE_MXFP4_E2M1 : d.dtype;
  return lmoe_fc2_combine_norm(d.T, d.E, d.K, d.d, d.L, d.tile_m, at, d.act, d.mx_experts ? d.act_scales : nullptr,
                               d.row_to_pair, d.tile_expert, wt, d.w2, d.mx_experts ? d.w2_scales : nullptr,
                               d.topk_weights, d.z, d.rows_cap, d.fc2_ws, d.fc2_ws_bytes, d.gamma, d.eps, d.dtype,
                               d.norm, s);
}

lmoe_status tail(const lmoe_layer_desc& d, bool fold, hipStream_t s) {
  if (fold)
    return lmoe_tail_shared_ws(d.T, d.L, d.H, d.I, nullptr, d.gamma, d.eps, d.w_up, d.shared_act, d.w_s2, d.dtype,
                               d.out, d.norm, d.tail_ws, d.tail_ws_bytes, s);
  return lmoe_tail(d.T, d.L, d.H, nullptr, d.gamma, d.eps, d.w_up, d.shared_out, d.dtype, d.out, d.norm, s);
}

// One step on `main` (and the layer's second stream). Returns the first failing call's
// status; the calls after it are not made.
lmoe_status step(lmoe_layer* ly, const void* X, hipStream_t main) {
  const lmoe_layer_desc& d = ly->d;
  const bool fold = folds(d);
  if (!d.shared_stream) {   // one stream: the shared FC1 in the front launch, its FC2 in the tail
    lmoe_status st = front(d, X, true, main);
    if (st == LMOE_OK) st = route(d, main);
    if (st == LMOE_OK) st = experts(d, main);
    if (st == LMOE_OK) st = tail(d, true, main);
    return st;
  }
  lmoe_status st = hip_ok(hipEventRecord(ly->ev_start, main));
  if (st == LMOE_OK) st = hip_ok(hipStreamWaitEvent(ly->side, ly->ev_start, 0));
  const bool fw = fork_wait(d);
  if (st == LMOE_OK && fw) st = hip_ok(hipEventRecord(ly->ev_fork, ly->side));
  if (st == LMOE_OK)
    st = lmoe_fc1_situ_capped(d.T, 1, 1, d.H, d.I, 16, d.dtype, X, nullptr, nullptr, nullptr, d.dtype, d.w_s1,
                              nullptr, d.beta, d.linear_beta, d.dtype, d.shared_act, nullptr, d.T, d.side_waves,
                              ly->side);
  if (st == LMOE_OK && fw) st = hip_ok(hipStreamWaitEvent(main, ly->ev_fork, 0));
  if (st == LMOE_OK && !fold)
    st = lmoe_fc2_combine(d.T, 1, 1, d.I, d.H, 16, d.dtype, d.shared_act, nullptr, nullptr, nullptr, d.dtype, d.w_s2,
                          nullptr, nullptr, d.dtype, d.shared_out, d.T, nullptr, 0, ly->side);
  if (st == LMOE_OK) st = hip_ok(hipEventRecord(ly->ev_shared, ly->side));
  if (st == LMOE_OK) st = front(d, X, false, main);
  if (st == LMOE_OK) st = route(d, main);
  if (st == LMOE_OK) st = experts(d, main);
  if (st == LMOE_OK) st = hip_ok(hipStreamWaitEvent(main, ly->ev_shared, 0));
  if (st == LMOE_OK) st = tail(d, fold, main);
  return st;
}

// The description's own checks: pointers, buffer and workspace sizes. The shape and dtype
// rules of the calls are checked by the zero-token calls in lmoe_layer_create.
lmoe_status check_desc(const lmoe_layer_desc& d) {
  if (d.T < 0 || d.H <= 0 || d.L <= 0 || d.E <= 0 || d.K <= 0 || d.d <= 0 || d.I <= 0) return LMOE_ERR_INVALID_ARG;
  if (!dense_dtype(d.dtype)) return LMOE_ERR_INVALID_ARG;
  if (d.routing != LMOE_ROUTE_SIGMOID && d.routing != LMOE_ROUTE_GROUPED && d.routing != LMOE_ROUTE_RENORMALIZE)
    return LMOE_ERR_INVALID_ARG;
  if (d.side_waves < 0 || d.fold_shared_fc2 < -1 || d.fold_shared_fc2 > 1) return LMOE_ERR_INVALID_ARG;
  if (!d.w_router || !d.w_down || !d.w1 || !d.w2 || !d.w_s1 || !d.w_s2 || !d.w_up) return LMOE_ERR_INVALID_ARG;
  if (d.mx_experts && (!d.w1_scales || !d.w2_scales)) return LMOE_ERR_INVALID_ARG;
  if (!d.logits || !d.topk_ids || !d.topk_weights || !d.expert_counts || !d.expert_offsets || !d.tile_offsets ||
      !d.row_to_pair || !d.tile_expert || !d.pair_to_row || !d.latent || !d.act || !d.z || !d.shared_act ||
      !d.norm || !d.out)
    return LMOE_ERR_INVALID_ARG;
  if (d.mx_experts && (!d.latent_q || !d.latent_scales || !d.act_scales)) return LMOE_ERR_INVALID_ARG;
  if (!folds(d) && !d.shared_out) return LMOE_ERR_INVALID_ARG;
  if (d.T == 0) return LMOE_OK;
  const int cap = lmoe_permute_rows_cap(d.T, d.E, d.K, d.tile_m);
  if (cap < 0) return LMOE_ERR_INVALID_ARG;
  if (d.rows_cap < cap || d.rows_cap % d.tile_m != 0) return LMOE_ERR_WORKSPACE;
  const size_t pw = lmoe_permute_workspace_bytes(d.T, d.E, d.K);
  if (pw > 0 && (!d.perm_ws || d.perm_ws_bytes < pw)) return LMOE_ERR_WORKSPACE;
  const size_t fw = lmoe_fc2_workspace_bytes(d.T, d.K, d.L);
  if (fw > 0 && (!d.fc2_ws || d.fc2_ws_bytes < fw)) return LMOE_ERR_WORKSPACE;
  // the front workspace the step's own front launch asks for (NULL: no split-K)
  const int N[3] = {d.E, d.L, d.I};
  const int situ[3] = {0, 0, 1};
  const size_t frw = lmoe_linear_multi_workspace_bytes(d.T, d.H, d.dtype, d.shared_stream ? 2 : 3, N, situ);
  if (d.front_ws && d.front_ws_bytes < frw) return LMOE_ERR_WORKSPACE;
  const size_t tw = folds(d) ? lmoe_tail_shared_workspace_bytes(d.T, d.L, d.H, d.I, d.dtype) : 0;
  if (d.tail_ws && d.tail_ws_bytes < tw) return LMOE_ERR_WORKSPACE;
  return LMOE_OK;
}

// Shape and dtype rules of every call the step makes, checked by calling each with no
// tokens (a zero-token call validates its arguments and enqueues nothing).
lmoe_status check_calls(const lmoe_layer_desc& d0) {
  lmoe_layer_desc d = d0;
  d.T = 0;
  lmoe_status st = front(d, d.latent, !d.shared_stream, nullptr);
  if (st == LMOE_OK) st = route(d, nullptr);
  if (st == LMOE_OK) st = experts(d, nullptr);
  if (st == LMOE_OK) st = tail(d, folds(d), nullptr);
  if (st == LMOE_OK && d.shared_stream) {
    st = lmoe_fc1_situ_capped(0, 1, 1, d.H, d.I, 16, d.dtype, d.latent, nullptr, nullptr, nullptr, d.dtype, d.w_s1,
                              nullptr, d.beta, d.linear_beta, d.dtype, d.shared_act, nullptr, 0, d.side_waves,
                              nullptr);
    if (st == LMOE_OK && !folds(d))
      st = lmoe_fc2_combine(0, 1, 1, d.I, d.H, 16, d.dtype, d.shared_act, nullptr, nullptr, nullptr, d.dtype, d.w_s2,
                            nullptr, nullptr, d.dtype, d.shared_out, 0, nullptr, 0, nullptr);
  }
  return st;
}

lmoe_status current_device_is(const lmoe_layer* ly) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LMOE_ERR_HIP;
  return dev == ly->device ? LMOE_OK : LMOE_ERR_INVALID_ARG;
}

}  // namespace

extern "C" {

size_t lmoe_layer_desc_bytes(void) { return sizeof(lmoe_layer_desc); }

lmoe_status lmoe_layer_create(const lmoe_layer_desc* desc, lmoe_layer** layer) {
  if (!desc || !layer) return LMOE_ERR_INVALID_ARG;
  *layer = nullptr;
  lmoe_status st = check_desc(*desc);
  if (st == LMOE_OK) st = check_calls(*desc);
  if (st != LMOE_OK) return st;
  lmoe_layer* ly = new (std::nothrow) lmoe_layer{};
  if (!ly) return LMOE_ERR_INVALID_ARG;
  ly->d = *desc;
  ly->side = desc->side_stream;
  if (hipGetDevice(&ly->device) != hipSuccess) {
    delete ly;
    return LMOE_ERR_HIP;
  }
  if (!ly->side && desc->shared_stream) {
    if (hipStreamCreateWithFlags(&ly->side, hipStreamNonBlocking) != hipSuccess) {   // default priority
      delete ly;
      return LMOE_ERR_HIP;
    }
    ly->own_side = true;
  }
  if (hipEventCreateWithFlags(&ly->ev_start, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&ly->ev_fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&ly->ev_shared, hipEventDisableTiming) != hipSuccess) {
    lmoe_layer_destroy(ly);
    return LMOE_ERR_HIP;
  }
  *layer = ly;
  return LMOE_OK;
}

lmoe_status lmoe_layer_forward(lmoe_layer* layer, const void* x, hipStream_t stream) {
  if (!layer) return LMOE_ERR_INVALID_ARG;
  if (layer->d.T == 0) return LMOE_OK;
  if (!x) return LMOE_ERR_INVALID_ARG;
  const lmoe_status st = current_device_is(layer);
  return st != LMOE_OK ? st : step(layer, x, stream);
}

lmoe_status lmoe_layer_capture(lmoe_layer* layer, const void* x, hipStream_t stream) {
  if (!layer || !x || !stream) return LMOE_ERR_INVALID_ARG;   // the legacy stream cannot be captured
  if (layer->d.T == 0) return LMOE_OK;
  lmoe_status st = current_device_is(layer);
  if (st != LMOE_OK) return st;
  if (hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal) != hipSuccess) return LMOE_ERR_HIP;
  st = step(layer, x, stream);
  hipGraph_t graph = nullptr;
  const hipError_t end = hipStreamEndCapture(stream, &graph);   // always ends the capture
  if (st == LMOE_OK && end != hipSuccess) st = LMOE_ERR_HIP;
  hipGraphExec_t exec = nullptr;
  if (st == LMOE_OK && hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) st = LMOE_ERR_HIP;
  if (graph) (void)hipGraphDestroy(graph);   // releases: nothing to report to the caller
  if (st != LMOE_OK) return st;
  if (layer->exec) (void)hipGraphExecDestroy(layer->exec);
  layer->exec = exec;
  return LMOE_OK;
}

lmoe_status lmoe_layer_replay(lmoe_layer* layer, hipStream_t stream) {
  if (!layer) return LMOE_ERR_INVALID_ARG;
  if (layer->d.T == 0) return LMOE_OK;
  if (!layer->exec) return LMOE_ERR_INVALID_ARG;
  const lmoe_status st = current_device_is(layer);
  return st != LMOE_OK ? st : (hipGraphLaunch(layer->exec, stream) == hipSuccess ? LMOE_OK : LMOE_ERR_HIP);
}

void lmoe_layer_destroy(lmoe_layer* layer) {
  if (!layer) return;
  // releases only: a failure here leaves nothing the caller could act on
  if (layer->exec) (void)hipGraphExecDestroy(layer->exec);
  if (layer->ev_start) (void)hipEventDestroy(layer->ev_start);
  if (layer->ev_fork) (void)hipEventDestroy(layer->ev_fork);
  if (layer->ev_shared) (void)hipEventDestroy(layer->ev_shared);
  if (layer->own_side && layer->side) (void)hipStreamDestroy(layer->side);
  delete layer;
}

}  // extern "C"
