// C ABI of liblmoe: argument validation and kernel dispatch. Declarations and the
// contract of every entry point are in include/lmoe.h.
#include <math.h>

#include "kernels.h"
#include "lmoe.h"

using namespace lmoe;

namespace {

bool dense_elt(lmoe_dtype t) { return t == LMOE_F32 || t == LMOE_BF16; }
Elt elt_of(lmoe_dtype t) { return t == LMOE_F32 ? Elt::F32 : Elt::BF16; }
int kchunk_of(lmoe_dtype t) { return t == LMOE_F32 ? 64 : 128; }
long esize_of(lmoe_dtype t) { return t == LMOE_F32 ? 4 : 2; }
// operand buffers are addressed with 32-bit byte offsets
bool fits32(long rows, long cols, lmoe_dtype t) { return rows * cols * esize_of(t) < 0xFFFFFFFFL; }
bool tile_ok(int tile_m) {
  return tile_m == 16 || tile_m == 32 || tile_m == 64 || tile_m == 128 || tile_m == 256;
}
lmoe_status hip_status(hipError_t e) { return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP; }
long rows_bound(long pairs, int E, int tile_m) {
  const long nonempty = pairs < E ? pairs : E;
  const long cap = pairs + nonempty * (tile_m - 1);
  return (cap + tile_m - 1) / tile_m * tile_m;
}
// Token-heavy bf16 calls go to the LDS-tiled kernel (128-row tiles); the rest stream the
// weights over 16-row tiles.
bool use_tiled_dense(long M, lmoe_dtype t) { return t == LMOE_BF16 && M >= 256; }
bool use_tiled_grouped(int tile_m, lmoe_dtype t) { return t == LMOE_BF16 && tile_m == 128; }
hipError_t run_gemm(const StreamGemm& g, lmoe_dtype t, bool tiled, int live, hipStream_t stream,
                    long target_waves = 0) {
  return tiled ? launch_tiled_gemm(g, stream) : launch_stream_gemm(g, elt_of(t), live, stream, target_waves);
}
// expected 16-row tiles holding rows: pairs / 16 plus one partial tile per touched expert
int live_tiles(long pairs, int E) {
  const long nonempty = pairs < E ? pairs : E;
  return (int)((pairs + 15) / 16 + nonempty);
}

}  // namespace

extern "C" {

int lmoe_abi_version(void) { return LMOE_ABI_VERSION; }

const char* lmoe_status_string(lmoe_status s) {
  switch (s) {
    case LMOE_OK: return "ok";
    case LMOE_ERR_INVALID_ARG: return "invalid argument";
    case LMOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case LMOE_ERR_WORKSPACE: return "workspace or capacity too small";
    case LMOE_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

lmoe_status lmoe_pack_weights(int batch, int N, int Kd, lmoe_dtype dtype, const void* src, void* dst,
                              hipStream_t stream) {
  if (batch < 0 || N < 0 || Kd < 0) return LMOE_ERR_INVALID_ARG;
  if (!dense_elt(dtype)) return dtype == LMOE_MXFP8_E4M3 ? LMOE_ERR_INVALID_ARG : LMOE_ERR_UNSUPPORTED;
  if (N % 16 != 0 || Kd % kchunk_of(dtype) != 0) return LMOE_ERR_UNSUPPORTED;
  if (batch == 0 || N == 0 || Kd == 0) return LMOE_OK;
  if (!src || !dst || src == dst) return LMOE_ERR_INVALID_ARG;
  return hip_status(launch_pack_weights(batch, N, Kd, (int)esize_of(dtype), src, dst, stream));
}

lmoe_status lmoe_pack_mxfp4_weights(int batch, int N, int Kd, const uint8_t* codes_src, const uint8_t* scales_src,
                                    uint8_t* codes_dst, uint8_t* scales_dst, hipStream_t stream) {
  if (batch < 0 || N < 0 || Kd < 0) return LMOE_ERR_INVALID_ARG;
  if (N % 16 != 0 || Kd % 512 != 0) return LMOE_ERR_UNSUPPORTED;
  if (batch == 0 || N == 0 || Kd == 0) return LMOE_OK;
  if (!codes_src || !scales_src || !codes_dst || !scales_dst || codes_src == codes_dst || scales_src == scales_dst)
    return LMOE_ERR_INVALID_ARG;
  return hip_status(launch_pack_mxfp4(batch, N, Kd, codes_src, scales_src, codes_dst, scales_dst, stream));
}

lmoe_status lmoe_linear(int M, int N, int Kd, lmoe_dtype x_dtype, const void* x, lmoe_dtype w_dtype,
                        const void* w, lmoe_dtype y_dtype, void* y, hipStream_t stream) {
  if (M < 0 || N <= 0 || Kd <= 0) return LMOE_ERR_INVALID_ARG;
  if (!dense_elt(x_dtype) || x_dtype != w_dtype || !dense_elt(y_dtype)) return LMOE_ERR_INVALID_ARG;
  if (Kd % kchunk_of(x_dtype) != 0 || N % 16 != 0) return LMOE_ERR_UNSUPPORTED;
  if (M == 0) return LMOE_OK;
  if (!x || !w || !y) return LMOE_ERR_INVALID_ARG;
  if (!fits32(M, Kd, x_dtype) || !fits32(N, Kd, w_dtype)) return LMOE_ERR_UNSUPPORTED;
  StreamGemm g{};
  g.a = x;
  g.a_bytes = (uint32_t)(M * (long)Kd * esize_of(x_dtype));
  g.lda = Kd;
  g.Kd = Kd;
  g.M = M;
  g.topk = 1;
  g.beta = 1.0f;
  g.nseg = 1;
  g.seg[0] = Seg{w, N, N, Epi::STORE, elt_of(y_dtype), y, N, 0, 0};
  return hip_status(run_gemm(g, x_dtype, use_tiled_dense(M, x_dtype), (M + 15) / 16, stream));
}

// Validates a lmoe_linear_multi call and fills g; LMOE_OK when a launch is needed.
static lmoe_status linear_multi_setup(int M, int Kd, lmoe_dtype x_dtype, const void* x, int n_proj, const int* N,
                                      const void* const* w, const lmoe_dtype* y_dtype, void* const* y,
                                      const int* situ, float beta, float linear_beta, bool check_ptrs,
                                      StreamGemm* out) {
  if (M < 0 || Kd <= 0 || n_proj < 1 || n_proj > 4 || !N) return LMOE_ERR_INVALID_ARG;
  if (check_ptrs && (!w || !y_dtype || !y)) return LMOE_ERR_INVALID_ARG;
  if (!dense_elt(x_dtype)) return LMOE_ERR_INVALID_ARG;
  bool any_situ = false;
  for (int i = 0; i < n_proj; ++i) {
    if (N[i] <= 0 || (check_ptrs && !dense_elt(y_dtype[i]))) return LMOE_ERR_INVALID_ARG;
    if (N[i] % 16 != 0) return LMOE_ERR_UNSUPPORTED;
    any_situ |= situ && situ[i];
  }
  if (any_situ && (!(beta > 0.0f) || !isfinite(beta) || isnan(linear_beta) || isinf(linear_beta)))
    return LMOE_ERR_INVALID_ARG;
  if (Kd % kchunk_of(x_dtype) != 0) return LMOE_ERR_UNSUPPORTED;
  if (M == 0) return LMOE_OK;
  if (check_ptrs && !x) return LMOE_ERR_INVALID_ARG;
  if (!fits32(M, Kd, x_dtype)) return LMOE_ERR_UNSUPPORTED;
  StreamGemm g{};
  g.a = x;
  g.a_bytes = (uint32_t)(M * (long)Kd * esize_of(x_dtype));
  g.lda = Kd;
  g.Kd = Kd;
  g.M = M;
  g.topk = 1;
  g.beta = beta;
  g.lbeta = linear_beta;
  g.nseg = n_proj;
  for (int i = 0; i < n_proj; ++i) {
    const bool si = situ && situ[i];
    if (check_ptrs && (!w[i] || !y[i])) return LMOE_ERR_INVALID_ARG;
    if (!fits32(si ? 2L * N[i] : N[i], Kd, x_dtype)) return LMOE_ERR_UNSUPPORTED;
    g.seg[i] = Seg{check_ptrs ? w[i] : nullptr, si ? 2 * N[i] : N[i], N[i], si ? Epi::SITU : Epi::STORE,
                   check_ptrs ? elt_of(y_dtype[i]) : Elt::F32, check_ptrs ? y[i] : nullptr, N[i], 0, 0};
  }
  *out = g;
  return LMOE_OK;
}

size_t lmoe_linear_multi_workspace_bytes(int M, int Kd, lmoe_dtype x_dtype, int n_proj, const int* N,
                                         const int* situ) {
  StreamGemm g{};
  if (M <= 0 || linear_multi_setup(M, Kd, x_dtype, nullptr, n_proj, N, nullptr, nullptr, nullptr, situ, 1.0f,
                                   0.0f, false, &g) != LMOE_OK)
    return 0;
  if (!use_tiled_dense(M, x_dtype)) return 0;
  return tiled_splitk_bytes(g, tiled_splitk(g));
}

lmoe_status lmoe_linear_multi_ws(int M, int Kd, lmoe_dtype x_dtype, const void* x, int n_proj, const int* N,
                                 const void* const* w, const lmoe_dtype* y_dtype, void* const* y, const int* situ,
                                 float beta, float linear_beta, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  StreamGemm g{};
  lmoe_status st = linear_multi_setup(M, Kd, x_dtype, x, n_proj, N, w, y_dtype, y, situ, beta, linear_beta, true,
                                      &g);
  if (st != LMOE_OK || M == 0) return st;
  const bool tiled = use_tiled_dense(M, x_dtype);
  if (tiled && workspace) {
    const int k = tiled_splitk(g);
    if (k > 1) {
      if (workspace_bytes < tiled_splitk_bytes(g, k)) return LMOE_ERR_WORKSPACE;
      g.part = static_cast<float*>(workspace);
      g.ksplit = k;
    }
  }
  return hip_status(run_gemm(g, x_dtype, tiled, (M + 15) / 16, stream));
}

lmoe_status lmoe_linear_multi(int M, int Kd, lmoe_dtype x_dtype, const void* x, int n_proj, const int* N,
                              const void* const* w, const lmoe_dtype* y_dtype, void* const* y, const int* situ,
                              float beta, float linear_beta, hipStream_t stream) {
  return lmoe_linear_multi_ws(M, Kd, x_dtype, x, n_proj, N, w, y_dtype, y, situ, beta, linear_beta, nullptr, 0,
                              stream);
}

lmoe_status lmoe_route(int T, int E, int K, const float* logits, const float* bias, float rsf, int renormalize,
                       int32_t* topk_ids, float* topk_weights, hipStream_t stream) {
  if (T < 0 || E < 1 || K < 1 || K > E || K > 64 || !isfinite(rsf)) return LMOE_ERR_INVALID_ARG;
  if (E > 1024) return LMOE_ERR_UNSUPPORTED;
  if (T == 0) return LMOE_OK;
  if (!logits || !topk_ids || !topk_weights) return LMOE_ERR_INVALID_ARG;
  return hip_status(launch_route(T, E, K, logits, bias, rsf, renormalize, topk_ids, topk_weights, stream));
}

lmoe_status lmoe_route_grouped(int T, int E, int K, int n_group, int topk_group, const float* logits,
                               const float* bias, float rsf, int renormalize, int32_t* topk_ids, float* topk_weights,
                               hipStream_t stream) {
  if (T < 0 || E < 1 || K < 1 || K > E || K > 64 || !isfinite(rsf)) return LMOE_ERR_INVALID_ARG;
  if (n_group < 1 || n_group > 64 || E % n_group != 0 || topk_group < 1 || topk_group > n_group ||
      K > topk_group * (E / n_group))
    return LMOE_ERR_INVALID_ARG;
  if (E > 1024) return LMOE_ERR_UNSUPPORTED;
  if (T == 0) return LMOE_OK;
  if (!logits || !topk_ids || !topk_weights) return LMOE_ERR_INVALID_ARG;
  if (n_group == 1 || topk_group == n_group)   // every expert competes: single-group routing
    return hip_status(launch_route(T, E, K, logits, bias, rsf, renormalize, topk_ids, topk_weights, stream));
  return hip_status(launch_route_grouped(T, E, K, n_group, topk_group, logits, bias, rsf, renormalize, topk_ids,
                                         topk_weights, stream));
}

lmoe_status lmoe_route_renormalize(int T, int E, int K, const float* logits, int32_t* topk_ids, float* topk_weights,
                                   hipStream_t stream) {
  if (T < 0 || E < 1 || K < 1 || K > E || K > 64) return LMOE_ERR_INVALID_ARG;
  if (E > 1024) return LMOE_ERR_UNSUPPORTED;
  if (T == 0) return LMOE_OK;
  if (!logits || !topk_ids || !topk_weights) return LMOE_ERR_INVALID_ARG;
  return hip_status(launch_route_renormalize(T, E, K, logits, topk_ids, topk_weights, stream));
}

size_t lmoe_permute_workspace_bytes(int T, int E, int K) {
  if (T <= 0 || E < 1 || K < 1) return 0;
  return permute_workspace_bytes((int)((long)T * K), E);
}

int lmoe_permute_rows_cap(int T, int E, int K, int tile_m) {
  if (T < 0 || E < 1 || K < 1 || !tile_ok(tile_m)) return -1;
  const long b = rows_bound((long)T * K, E, tile_m);
  return b > 0x7FFFFFFFL ? -1 : (int)b;
}

lmoe_status lmoe_permute(int T, int E, int K, int tile_m, const int32_t* topk_ids, int32_t* expert_counts,
                         int32_t* expert_offsets, int32_t* tile_offsets, int32_t* row_to_pair, int32_t* tile_expert,
                         int32_t* pair_to_row, int rows_cap, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (T < 0 || E < 1 || K < 1 || K > E || K > 64 || !tile_ok(tile_m)) return LMOE_ERR_INVALID_ARG;
  if (E > 1024) return LMOE_ERR_UNSUPPORTED;
  if ((long)T * K > 0x3FFFFFFFL) return LMOE_ERR_UNSUPPORTED;
  if (T == 0) return LMOE_OK;
  if (!topk_ids || !expert_counts || !expert_offsets || !tile_offsets || !row_to_pair || !tile_expert ||
      !pair_to_row)
    return LMOE_ERR_INVALID_ARG;
  const long npairs = (long)T * K;
  if (rows_cap < rows_bound(npairs, E, tile_m) || rows_cap % tile_m != 0) return LMOE_ERR_WORKSPACE;
  const size_t need = permute_workspace_bytes((int)npairs, E);
  if (need > 0 && (!workspace || workspace_bytes < need)) return LMOE_ERR_WORKSPACE;
  return hip_status(launch_permute((int)npairs, E, tile_m, rows_cap / tile_m, topk_ids, expert_counts,
                                   expert_offsets, tile_offsets, row_to_pair, tile_expert, pair_to_row, workspace,
                                   stream));
}

size_t lmoe_permute_noalloc_max_bytes(void) { return PERMUTE_SCRATCH_BYTES; }

lmoe_status lmoe_permute_noalloc(int T, int E, int K, int tile_m, const int32_t* topk_ids, int32_t* expert_counts,
                                 int32_t* expert_offsets, int32_t* tile_offsets, int32_t* row_to_pair,
                                 int32_t* tile_expert, int32_t* pair_to_row, int rows_cap, hipStream_t stream) {
  if (T < 0 || E < 1 || K < 1 || K > E || K > 64 || !tile_ok(tile_m)) return LMOE_ERR_INVALID_ARG;
  if (E > 1024) return LMOE_ERR_UNSUPPORTED;
  if ((long)T * K > 0x3FFFFFFFL) return LMOE_ERR_UNSUPPORTED;
  if (T == 0) return LMOE_OK;
  if (!topk_ids || !expert_counts || !expert_offsets || !tile_offsets || !row_to_pair || !tile_expert ||
      !pair_to_row)
    return LMOE_ERR_INVALID_ARG;
  const long npairs = (long)T * K;
  if (rows_cap < rows_bound(npairs, E, tile_m) || rows_cap % tile_m != 0) return LMOE_ERR_WORKSPACE;
  if (permute_workspace_bytes((int)npairs, E) > PERMUTE_SCRATCH_BYTES) return LMOE_ERR_WORKSPACE;
  // the scratch address is the current device's: the stream must belong to that device
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return LMOE_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return LMOE_ERR_HIP;
    if ((int)sdev != cur) return LMOE_ERR_INVALID_ARG;
  }
  void* scratch_ptr = nullptr;
  if (permute_scratch(&scratch_ptr) != hipSuccess) return LMOE_ERR_HIP;
  return hip_status(launch_permute((int)npairs, E, tile_m, rows_cap / tile_m, topk_ids, expert_counts,
                                   expert_offsets, tile_offsets, row_to_pair, tile_expert, pair_to_row, scratch_ptr,
                                   stream));
}

lmoe_status lmoe_route_permute(int T, int E, int K, const float* logits, const float* bias, float rsf,
                               int renormalize, int32_t* topk_ids, float* topk_weights, int tile_m,
                               int32_t* expert_counts, int32_t* expert_offsets, int32_t* tile_offsets,
                               int32_t* row_to_pair, int32_t* tile_expert, int32_t* pair_to_row, int rows_cap,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // the checks of lmoe_route, then those of lmoe_permute
  if (T < 0 || E < 1 || K < 1 || K > E || K > 64 || !isfinite(rsf) || !tile_ok(tile_m)) return LMOE_ERR_INVALID_ARG;
  if (E > 1024) return LMOE_ERR_UNSUPPORTED;
  if ((long)T * K > 0x3FFFFFFFL) return LMOE_ERR_UNSUPPORTED;
  if (T == 0) return LMOE_OK;
  if (!logits || !topk_ids || !topk_weights || !expert_counts || !expert_offsets || !tile_offsets ||
      !row_to_pair || !tile_expert || !pair_to_row)
    return LMOE_ERR_INVALID_ARG;
  const long npairs = (long)T * K;
  if (rows_cap < rows_bound(npairs, E, tile_m) || rows_cap % tile_m != 0) return LMOE_ERR_WORKSPACE;
  const size_t need = permute_workspace_bytes((int)npairs, E);
  if (need > 0 && (!workspace || workspace_bytes < need)) return LMOE_ERR_WORKSPACE;
  return hip_status(launch_route_permute(T, E, K, logits, bias, rsf, renormalize, topk_ids, topk_weights, tile_m,
                                         rows_cap / tile_m, expert_counts, expert_offsets, tile_offsets,
                                         row_to_pair, tile_expert, pair_to_row, workspace, stream));
}

lmoe_status lmoe_quant_mxfp8(int rows, int cols, lmoe_dtype in_dtype, const void* in, uint8_t* codes,
                             uint8_t* scales, hipStream_t stream) {
  if (rows < 0 || cols <= 0 || !dense_elt(in_dtype)) return LMOE_ERR_INVALID_ARG;
  if (cols % 32 != 0) return LMOE_ERR_UNSUPPORTED;
  if (rows == 0) return LMOE_OK;
  if (!in || !codes || !scales) return LMOE_ERR_INVALID_ARG;
  return hip_status(launch_quant_mxfp8(rows, cols, elt_of(in_dtype), in, codes, scales, stream));
}

// Common checks of the grouped expert GEMMs; returns LMOE_OK when the mode is valid.
static lmoe_status check_grouped(int T, int E, int K, int tile_m, const int32_t* row_to_pair,
                                 const int32_t* tile_expert, int rows_cap, bool* dense) {
  if (T < 0 || E < 1 || K < 1 || K > 64) return LMOE_ERR_INVALID_ARG;
  if (!row_to_pair && !tile_expert) {
    if (E != 1 || K != 1 || rows_cap < T) return LMOE_ERR_INVALID_ARG;
    *dense = true;
    return LMOE_OK;
  }
  if (!row_to_pair || !tile_expert || !tile_ok(tile_m)) return LMOE_ERR_INVALID_ARG;
  if (rows_cap % tile_m != 0 || rows_cap < rows_bound((long)T * K, E, tile_m)) return LMOE_ERR_WORKSPACE;
  *dense = false;
  return LMOE_OK;
}

static lmoe_status fc1_situ_impl(int T, int E, int K, int in_dim, int d, int tile_m, lmoe_dtype a_dtype,
                                 const void* a, const uint8_t* a_scale, const int32_t* row_to_pair,
                                 const int32_t* tile_expert, lmoe_dtype w_dtype, const void* w1,
                                 const uint8_t* w1_scale, float beta, float linear_beta, lmoe_dtype act_dtype,
                                 void* act, uint8_t* act_scale, int rows_cap, long target_waves,
                                 hipStream_t stream) {
  bool dense = false;
  lmoe_status st = check_grouped(T, E, K, tile_m, row_to_pair, tile_expert, rows_cap, &dense);
  if (st != LMOE_OK) return st;
  if (in_dim <= 0 || d <= 0) return LMOE_ERR_INVALID_ARG;
  if (!(beta > 0.0f) || !isfinite(beta) || isnan(linear_beta) || isinf(linear_beta)) return LMOE_ERR_INVALID_ARG;
  const bool mx = a_dtype == LMOE_MXFP8_E4M3 || w_dtype == LMOE_MXFP4_E2M1;
  if (mx) {
    if (a_dtype != LMOE_MXFP8_E4M3 || w_dtype != LMOE_MXFP4_E2M1 || act_dtype != LMOE_MXFP8_E4M3)
      return LMOE_ERR_INVALID_ARG;
    if (dense || in_dim % 512 != 0 || d % 32 != 0) return LMOE_ERR_UNSUPPORTED;
    if (T == 0) return LMOE_OK;
    if (!a || !a_scale || !w1 || !w1_scale || !act || !act_scale) return LMOE_ERR_INVALID_ARG;
    if ((long)T * in_dim >= 0xFFFFFFFFL || 2L * d * in_dim / 2 >= 0xFFFFFFFFL) return LMOE_ERR_UNSUPPORTED;
    StreamGemm g{};
    g.a = a;
    g.a_bytes = (uint32_t)((long)T * in_dim);
    g.a_scale = a_scale;
    g.a_scale_bytes = (uint32_t)((long)T * in_dim / 32);
    g.lda = in_dim;
    g.Kd = in_dim;
    g.M = rows_cap;
    g.row_to_pair = row_to_pair;
    g.tile_expert = tile_expert;
    g.tile_m = tile_m;
    g.topk = K;
    g.a_by_row = 0;
    g.beta = beta;
    g.lbeta = linear_beta;
    g.w_scale = w1_scale;
    g.out_scale = act_scale;
    g.nseg = 1;
    g.seg[0] = Seg{w1, 2 * d, d, Epi::SITU_MX, Elt::F32, act, d, 0, 0};
    return hip_status(launch_stream_gemm_mx(g, live_tiles((long)T * K, E), stream));
  }
  if (!dense_elt(a_dtype) || a_dtype != w_dtype || act_dtype != a_dtype) return LMOE_ERR_INVALID_ARG;
  if (in_dim % kchunk_of(a_dtype) != 0 || d % 16 != 0) return LMOE_ERR_UNSUPPORTED;
  if (T == 0) return LMOE_OK;
  if (!a || !w1 || !act) return LMOE_ERR_INVALID_ARG;
  if (!fits32(T, in_dim, a_dtype) || !fits32(2L * d, in_dim, w_dtype)) return LMOE_ERR_UNSUPPORTED;
  StreamGemm g{};
  g.weights_once = T <= 16;   // an expert then holds at most 16 rows: one row tile
  g.a = a;
  g.a_bytes = (uint32_t)((long)T * in_dim * esize_of(a_dtype));
  g.lda = in_dim;
  g.Kd = in_dim;
  g.M = dense ? T : rows_cap;
  g.row_to_pair = dense ? nullptr : row_to_pair;
  g.tile_expert = dense ? nullptr : tile_expert;
  g.tile_m = tile_m;
  g.topk = K;
  g.a_by_row = 0;
  g.beta = beta;
  g.lbeta = linear_beta;
  g.nseg = 1;
  g.seg[0] = Seg{w1, 2 * d, d, Epi::SITU, elt_of(act_dtype), act, d, 0, 0};
  const int live = dense ? (T + 15) / 16 : live_tiles((long)T * K, E);
  const bool tiled = dense ? use_tiled_dense(T, a_dtype) : use_tiled_grouped(tile_m, a_dtype);
  return hip_status(run_gemm(g, a_dtype, tiled, live, stream, target_waves));
}

lmoe_status lmoe_fc1_situ(int T, int E, int K, int in_dim, int d, int tile_m, lmoe_dtype a_dtype, const void* a,
                          const uint8_t* a_scale, const int32_t* row_to_pair, const int32_t* tile_expert,
                          lmoe_dtype w_dtype, const void* w1, const uint8_t* w1_scale, float beta, float linear_beta,
                          lmoe_dtype act_dtype, void* act, uint8_t* act_scale, int rows_cap, hipStream_t stream) {
  return fc1_situ_impl(T, E, K, in_dim, d, tile_m, a_dtype, a, a_scale, row_to_pair, tile_expert, w_dtype, w1,
                       w1_scale, beta, linear_beta, act_dtype, act, act_scale, rows_cap, 0, stream);
}

lmoe_status lmoe_fc1_situ_capped(int T, int E, int K, int in_dim, int d, int tile_m, lmoe_dtype a_dtype,
                                 const void* a, const uint8_t* a_scale, const int32_t* row_to_pair,
                                 const int32_t* tile_expert, lmoe_dtype w_dtype, const void* w1,
                                 const uint8_t* w1_scale, float beta, float linear_beta, lmoe_dtype act_dtype,
                                 void* act, uint8_t* act_scale, int rows_cap, int max_waves, hipStream_t stream) {
  if (max_waves < 0) return LMOE_ERR_INVALID_ARG;
  return fc1_situ_impl(T, E, K, in_dim, d, tile_m, a_dtype, a, a_scale, row_to_pair, tile_expert, w_dtype, w1,
                       w1_scale, beta, linear_beta, act_dtype, act, act_scale, rows_cap, max_waves, stream);
}

size_t lmoe_fc2_workspace_bytes(int T, int K, int out_dim) {
  if (T <= 0 || K <= 1 || out_dim <= 0) return 0;
  return (size_t)T * K * out_dim * sizeof(float);
}

// FC2 + combine; with norm_out != NULL the combined fp32 rows are also RMS-normalized into
// norm_out (norm_dtype, with gamma of that dtype) by the same kernel that sums them.
static lmoe_status fc2_combine_impl(int T, int E, int K, int d, int out_dim, int tile_m, lmoe_dtype act_dtype,
                                    const void* act, const uint8_t* act_scale, const int32_t* row_to_pair,
                                    const int32_t* tile_expert, lmoe_dtype w_dtype, const void* w2,
                                    const uint8_t* w2_scale, const float* topk_weights, lmoe_dtype out_dtype,
                                    void* out, int rows_cap, void* workspace, size_t workspace_bytes,
                                    const void* gamma, float eps, lmoe_dtype norm_dtype, void* norm_out,
                                    hipStream_t stream) {
  const bool norm = norm_out != nullptr;
  auto finish = [&](hipError_t err) -> lmoe_status {   // combine (K > 1) and / or RMSNorm
    if (err != hipSuccess) return LMOE_ERR_HIP;
    if (K > 1 && norm)
      err = launch_combine_norm(T, K, out_dim, (const float*)workspace, (float*)out, gamma, eps, elt_of(norm_dtype),
                                norm_out, stream);
    else if (K > 1)
      err = launch_combine(T, K, out_dim, (const float*)workspace, elt_of(out_dtype), out, stream);
    else if (norm)
      err = launch_rmsnorm(T, out_dim, (const float*)out, gamma, eps, elt_of(norm_dtype), norm_out, stream);
    return hip_status(err);
  };
  bool dense = false;
  lmoe_status st = check_grouped(T, E, K, tile_m, row_to_pair, tile_expert, rows_cap, &dense);
  if (st != LMOE_OK) return st;
  if (d <= 0 || out_dim <= 0 || !dense_elt(out_dtype)) return LMOE_ERR_INVALID_ARG;
  const bool mx = act_dtype == LMOE_MXFP8_E4M3 || w_dtype == LMOE_MXFP4_E2M1;
  if (mx) {
    if (act_dtype != LMOE_MXFP8_E4M3 || w_dtype != LMOE_MXFP4_E2M1) return LMOE_ERR_INVALID_ARG;
    if (dense || d % 512 != 0 || out_dim % 64 != 0) return LMOE_ERR_UNSUPPORTED;
    if (T == 0) return LMOE_OK;
    if (!act || !act_scale || !w2 || !w2_scale || !out) return LMOE_ERR_INVALID_ARG;
    if (K > 1 && (!workspace || workspace_bytes < lmoe_fc2_workspace_bytes(T, K, out_dim))) return LMOE_ERR_WORKSPACE;
    if ((long)rows_cap * d >= 0xFFFFFFFFL || (long)out_dim * d / 2 >= 0xFFFFFFFFL) return LMOE_ERR_UNSUPPORTED;
    StreamGemm g{};
    g.a = act;
    g.a_bytes = (uint32_t)((long)rows_cap * d);
    g.a_scale = act_scale;
    g.a_scale_bytes = (uint32_t)((long)rows_cap * d / 32);
    g.lda = d;
    g.Kd = d;
    g.M = rows_cap;
    g.row_to_pair = row_to_pair;
    g.tile_expert = tile_expert;
    g.tile_m = tile_m;
    g.topk = K;
    g.a_by_row = 1;
    g.pair_w = topk_weights;
    g.beta = 1.0f;
    g.w_scale = w2_scale;
    g.nseg = 1;
    if (K == 1)
      g.seg[0] = Seg{w2, out_dim, out_dim, Epi::TOKEN, elt_of(out_dtype), out, out_dim, 0, 0};
    else
      g.seg[0] = Seg{w2, out_dim, out_dim, Epi::PAIR, Elt::F32, workspace, out_dim, 0, 0};
    return finish(launch_stream_gemm_mx(g, live_tiles((long)T * K, E), stream));
  }
  if (!dense_elt(act_dtype) || act_dtype != w_dtype) return LMOE_ERR_INVALID_ARG;
  if (d % kchunk_of(act_dtype) != 0 || out_dim % 16 != 0) return LMOE_ERR_UNSUPPORTED;
  if (T == 0) return LMOE_OK;
  if (!act || !w2 || !out) return LMOE_ERR_INVALID_ARG;
  if (K > 1 && (!workspace || workspace_bytes < lmoe_fc2_workspace_bytes(T, K, out_dim))) return LMOE_ERR_WORKSPACE;
  const long act_rows = dense ? T : rows_cap;
  if (!fits32(act_rows, d, act_dtype) || !fits32(out_dim, d, w_dtype)) return LMOE_ERR_UNSUPPORTED;
  StreamGemm g{};
  g.weights_once = T <= 16;   // an expert then holds at most 16 rows: one row tile
  g.a = act;
  g.a_bytes = (uint32_t)(act_rows * d * esize_of(act_dtype));
  g.lda = d;
  g.Kd = d;
  g.M = dense ? T : rows_cap;
  g.row_to_pair = dense ? nullptr : row_to_pair;
  g.tile_expert = dense ? nullptr : tile_expert;
  g.tile_m = tile_m;
  g.topk = K;
  g.a_by_row = 1;
  g.pair_w = topk_weights;
  g.beta = 1.0f;
  g.nseg = 1;
  if (K == 1)
    g.seg[0] = Seg{w2, out_dim, out_dim, Epi::TOKEN, elt_of(out_dtype), out, out_dim, 0, 0};
  else
    g.seg[0] = Seg{w2, out_dim, out_dim, Epi::PAIR, Elt::F32, workspace, out_dim, 0, 0};
  const int live = dense ? (T + 15) / 16 : live_tiles((long)T * K, E);
  const bool tiled = dense ? use_tiled_dense(T, act_dtype) : use_tiled_grouped(tile_m, act_dtype);
  return finish(run_gemm(g, act_dtype, tiled, live, stream));
}

lmoe_status lmoe_fc2_combine(int T, int E, int K, int d, int out_dim, int tile_m, lmoe_dtype act_dtype,
                             const void* act, const uint8_t* act_scale, const int32_t* row_to_pair,
                             const int32_t* tile_expert, lmoe_dtype w_dtype, const void* w2,
                             const uint8_t* w2_scale, const float* topk_weights, lmoe_dtype out_dtype, void* out,
                             int rows_cap, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fc2_combine_impl(T, E, K, d, out_dim, tile_m, act_dtype, act, act_scale, row_to_pair, tile_expert, w_dtype,
                          w2, w2_scale, topk_weights, out_dtype, out, rows_cap, workspace, workspace_bytes, nullptr,
                          0.0f, LMOE_F32, nullptr, stream);
}

lmoe_status lmoe_fc2_combine_norm(int T, int E, int K, int d, int out_dim, int tile_m, lmoe_dtype act_dtype,
                                  const void* act, const uint8_t* act_scale, const int32_t* row_to_pair,
                                  const int32_t* tile_expert, lmoe_dtype w_dtype, const void* w2,
                                  const uint8_t* w2_scale, const float* topk_weights, float* z, int rows_cap,
                                  void* workspace, size_t workspace_bytes, const void* gamma, float eps,
                                  lmoe_dtype norm_dtype, void* norm_out, hipStream_t stream) {
  if (!dense_elt(norm_dtype) || !(eps >= 0.0f) || !isfinite(eps)) return LMOE_ERR_INVALID_ARG;
  if (out_dim % 4 != 0) return LMOE_ERR_UNSUPPORTED;
  if (T > 0 && !norm_out) return LMOE_ERR_INVALID_ARG;
  if (T > 0 && (void*)z == norm_out) return LMOE_ERR_INVALID_ARG;
  return fc2_combine_impl(T, E, K, d, out_dim, tile_m, act_dtype, act, act_scale, row_to_pair, tile_expert, w_dtype,
                          w2, w2_scale, topk_weights, LMOE_F32, z, rows_cap, workspace, workspace_bytes, gamma, eps,
                          norm_dtype, T > 0 ? norm_out : nullptr, stream);
}

lmoe_status lmoe_tail(int T, int L, int H, const float* latent, const void* gamma, float eps, const void* w_up,
                      const void* shared, lmoe_dtype io_dtype, void* out, void* norm_out, hipStream_t stream) {
  if (T < 0 || L <= 0 || H <= 0) return LMOE_ERR_INVALID_ARG;
  if (!dense_elt(io_dtype) || !(eps >= 0.0f) || !isfinite(eps)) return LMOE_ERR_INVALID_ARG;
  if (L % kchunk_of(io_dtype) != 0 || H % 16 != 0) return LMOE_ERR_UNSUPPORTED;
  if (T == 0) return LMOE_OK;
  if (!w_up || !out || !norm_out) return LMOE_ERR_INVALID_ARG;
  if (!fits32(T, L, io_dtype) || !fits32(H, L, io_dtype)) return LMOE_ERR_UNSUPPORTED;
  if (latent) {   // NULL: norm_out already holds the normalized latent
    hipError_t err = launch_rmsnorm(T, L, latent, gamma, eps, elt_of(io_dtype), norm_out, stream);
    if (err != hipSuccess) return LMOE_ERR_HIP;
  }
  StreamGemm g{};
  g.a = norm_out;
  g.a_bytes = (uint32_t)((long)T * L * esize_of(io_dtype));
  g.lda = L;
  g.Kd = L;
  g.M = T;
  g.topk = 1;
  g.add = shared;
  g.beta = 1.0f;
  g.nseg = 1;
  g.seg[0] = Seg{w_up, H, H, Epi::ADD, elt_of(io_dtype), out, H, 0, 0};
  return hip_status(run_gemm(g, io_dtype, use_tiled_dense(T, io_dtype), (T + 15) / 16, stream));
}

// The tiled two-phase GEMM of the token-heavy tail: out = shared_act @ w_s2^T +
// norm_out @ w_up^T, one set of fp32 accumulators.
static StreamGemm tail_shared_gemm(int T, int L, int H, int I, const void* w_up, const void* shared_act,
                                   const void* w_s2, lmoe_dtype io_dtype, void* out, const void* norm_out) {
  StreamGemm g{};
  g.a = shared_act;
  g.a_bytes = (uint32_t)((long)T * I * esize_of(io_dtype));
  g.lda = I;
  g.Kd = I;
  g.a1 = norm_out;
  g.a1_bytes = (uint32_t)((long)T * L * esize_of(io_dtype));
  g.lda1 = L;
  g.Kd1 = L;
  g.w1 = w_up;
  g.M = T;
  g.topk = 1;
  g.beta = 1.0f;
  g.nseg = 1;
  g.seg[0] = Seg{w_s2, H, H, Epi::STORE, elt_of(io_dtype), out, H, 0, 0};
  return g;
}

// Output columns [c0, c0 + nc) of the tail GEMM: the weight rows of both phases (packed
// in 16-row groups, so a row offset is a byte offset) and the output columns, row pitch H.
static StreamGemm tail_columns(StreamGemm g, int c0, int nc, int L, int I, int H, lmoe_dtype io_dtype) {
  const size_t es = (size_t)esize_of(io_dtype);
  if (g.seg[0].w) g.seg[0].w = static_cast<const char*>(g.seg[0].w) + (size_t)c0 * I * es;
  if (g.w1) g.w1 = static_cast<const char*>(g.w1) + (size_t)c0 * L * es;
  if (g.seg[0].out) g.seg[0].out = static_cast<char*>(g.seg[0].out) + (size_t)c0 * es;
  g.seg[0].n_total = nc;
  g.seg[0].n_out = nc;
  g.seg[0].ldo = H;
  return g;
}

static lmoe_status tail_shared_impl(int T, int L, int H, int I, const float* latent, const void* gamma, float eps,
                                    const void* w_up, const void* shared_act, const void* w_s2,
                                    lmoe_dtype io_dtype, void* out, void* norm_out, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || L <= 0 || H <= 0 || I <= 0) return LMOE_ERR_INVALID_ARG;
  if (!dense_elt(io_dtype) || !(eps >= 0.0f) || !isfinite(eps)) return LMOE_ERR_INVALID_ARG;
  if (L % kchunk_of(io_dtype) != 0 || I % kchunk_of(io_dtype) != 0 || H % 16 != 0) return LMOE_ERR_UNSUPPORTED;
  if (T == 0) return LMOE_OK;
  if (!w_up || !shared_act || !w_s2 || !out || !norm_out) return LMOE_ERR_INVALID_ARG;
  if (out == shared_act || out == norm_out) return LMOE_ERR_INVALID_ARG;
  if (!fits32(T, L, io_dtype) || !fits32(T, I, io_dtype) || !fits32(H, L, io_dtype) || !fits32(H, I, io_dtype))
    return LMOE_ERR_UNSUPPORTED;
  hipError_t err = hipSuccess;
  if (latent) {   // NULL: norm_out already holds the normalized latent
    err = launch_rmsnorm(T, L, latent, gamma, eps, elt_of(io_dtype), norm_out, stream);
    if (err != hipSuccess) return LMOE_ERR_HIP;
  }
  if (use_tiled_dense(T, io_dtype)) {
    // token-heavy: one tiled GEMM with two K phases, out = round(shared_act w_s2^T +
    // norm_out w_up^T): the shared-expert FC2 and the up projection accumulate into the
    // same fp32 tiles (the shared output is not rounded on its own here); with a
    // workspace, split-K when the tiles alone would leave CUs idle: for the whole GEMM
    // when it has less than a round of tiles, else for the columns past the last whole
    // round of tiles, in a second launch (T = 8192, H = 7168: 768 tiles at full K, then
    // 128 tiles in two K slices, rather than 896 tiles of which the last 128 run alone)
    StreamGemm g = tail_shared_gemm(T, L, H, I, w_up, shared_act, w_s2, io_dtype, out, norm_out);
    if (!tiled_dual_ok(g)) return LMOE_ERR_UNSUPPORTED;
    if (workspace) {
      const int c1 = tiled_round_cols(T, H);
      if (c1 < H) {
        StreamGemm g2 = tail_columns(g, c1, H - c1, L, I, H, io_dtype);
        const int k = tiled_splitk(g2);
        if (k > 1) {
          if (workspace_bytes < tiled_splitk_bytes(g2, k)) return LMOE_ERR_WORKSPACE;
          g2.part = static_cast<float*>(workspace);
          g2.ksplit = k;
        }
        const hipError_t e1 = launch_tiled_gemm(tail_columns(g, 0, c1, L, I, H, io_dtype), stream);
        if (e1 != hipSuccess) return hip_status(e1);
        return hip_status(launch_tiled_gemm(g2, stream));
      }
      const int k = tiled_splitk(g);
      if (k > 1) {
        if (workspace_bytes < tiled_splitk_bytes(g, k)) return LMOE_ERR_WORKSPACE;
        g.part = static_cast<float*>(workspace);
        g.ksplit = k;
      }
    }
    return hip_status(launch_tiled_gemm(g, stream));
  }
  StreamGemm g{};
  g.a = shared_act;                  // phase 0: shared-expert FC2, rounded like a stored tensor
  g.a_bytes = (uint32_t)((long)T * I * esize_of(io_dtype));
  g.lda = I;
  g.Kd = I;
  g.a1 = norm_out;                   // phase 1: up projection of the normalized latent
  g.a1_bytes = (uint32_t)((long)T * L * esize_of(io_dtype));
  g.lda1 = L;
  g.Kd1 = L;
  g.w1 = w_up;
  g.M = T;
  g.topk = 1;
  g.beta = 1.0f;
  g.nseg = 1;
  g.seg[0] = Seg{w_s2, H, H, Epi::ADD2, elt_of(io_dtype), out, H, 0, 0};
  return hip_status(launch_stream_gemm(g, elt_of(io_dtype), (T + 15) / 16, stream));
}

lmoe_status lmoe_tail_shared(int T, int L, int H, int I, const float* latent, const void* gamma, float eps,
                             const void* w_up, const void* shared_act, const void* w_s2, lmoe_dtype io_dtype,
                             void* out, void* norm_out, hipStream_t stream) {
  return tail_shared_impl(T, L, H, I, latent, gamma, eps, w_up, shared_act, w_s2, io_dtype, out, norm_out, nullptr,
                          0, stream);
}

size_t lmoe_tail_shared_workspace_bytes(int T, int L, int H, int I, lmoe_dtype io_dtype) {
  if (T <= 0 || L <= 0 || H <= 0 || I <= 0 || !dense_elt(io_dtype) || !use_tiled_dense(T, io_dtype)) return 0;
  if (L % kchunk_of(io_dtype) != 0 || I % kchunk_of(io_dtype) != 0 || H % 16 != 0) return 0;
  const StreamGemm g = tail_shared_gemm(T, L, H, I, nullptr, nullptr, nullptr, io_dtype, nullptr, nullptr);
  const int c1 = tiled_round_cols(T, H);
  if (c1 < H) {
    const StreamGemm g2 = tail_columns(g, c1, H - c1, L, I, H, io_dtype);
    return tiled_splitk_bytes(g2, tiled_splitk(g2));
  }
  return tiled_splitk_bytes(g, tiled_splitk(g));
}

lmoe_status lmoe_tail_shared_ws(int T, int L, int H, int I, const float* latent, const void* gamma, float eps,
                                const void* w_up, const void* shared_act, const void* w_s2, lmoe_dtype io_dtype,
                                void* out, void* norm_out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return tail_shared_impl(T, L, H, I, latent, gamma, eps, w_up, shared_act, w_s2, io_dtype, out, norm_out,
                          workspace, workspace_bytes, stream);
}

lmoe_status lmoe_situ_masked(int E, int T_max, int d, lmoe_dtype dtype, const void* in,
                             const int32_t* expert_num_tokens, float beta, float linear_beta, void* out,
                             hipStream_t stream) {
  if (E < 0 || T_max < 0 || d <= 0 || !dense_elt(dtype)) return LMOE_ERR_INVALID_ARG;
  if (!(beta > 0.0f) || !isfinite(beta) || isnan(linear_beta) || isinf(linear_beta)) return LMOE_ERR_INVALID_ARG;
  if (d % 8 != 0) return LMOE_ERR_UNSUPPORTED;
  if (E == 0 || T_max == 0) return LMOE_OK;
  if (!in || !expert_num_tokens || !out) return LMOE_ERR_INVALID_ARG;
  return hip_status(
      launch_situ_masked(E, T_max, d, elt_of(dtype), in, expert_num_tokens, beta, linear_beta, out, stream));
}

}  // extern "C"
