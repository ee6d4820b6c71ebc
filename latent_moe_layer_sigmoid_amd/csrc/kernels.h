// Host-side launchers of the gfx950 kernels (internal to liblmoe).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lmoe {

enum class Elt : int { F32 = 0, BF16 = 1 };

// Epilogue of the weight-streaming GEMM.
enum class Epi : int {
  STORE = 0,    // y[row, n] = acc                                    (out_elt)
  SITU = 1,     // y[row, j] = SituGLU(acc[j], acc[d + j])             (out_elt)
  PAIR = 2,     // ws[pair, n] = w[pair] * acc                         (fp32, combined afterwards)
  TOKEN = 3,    // out[token, n] = w[pair] * acc                       (out_elt; K == 1)
  ADD = 4,      // out[row, n] = add[row, n] + acc                     (out_elt)
  ADD2 = 5,     // out[row, n] = round(acc) + acc1 (second K phase)    (out_elt)
  SITU_MX = 6   // SituGLU, then MXFP8 requant per 32 outputs (codes + e8m0 scales)
};

// One group of output columns with its own weight and epilogue. Several segments that
// share the activation rows run in one launch.
struct Seg {
  const void* w;       // packed weights [E or 1][n_total][Kd]
  int n_total;         // rows of one expert's weight matrix
  int n_out;           // output columns (SituGLU: d, the weight has 2d rows)
  Epi epi;
  Elt out_elt;
  void* out;
  int ldo;
  int blocks;          // filled by the launcher
  int block0;          // filled by the launcher
};

struct StreamGemm {
  // A operand: rows of `a` ([*, lda] elements). Grouped mode gathers token rows
  // (row_to_pair / K) or, with a_by_row, the row itself; dense mode uses row r < M.
  const void* a;
  uint32_t a_bytes;          // size of the `a` buffer (hardware range check of the loads)
  int lda;
  int Kd;
  // optional second K phase (dense, one segment): acc1 = a1 @ w1^T, epilogue ADD2
  const void* a1;
  uint32_t a1_bytes;
  int lda1;
  int Kd1;
  const void* w1;
  int M;                     // dense: rows; grouped: rows_cap
  const int32_t* row_to_pair;  // NULL = dense
  const int32_t* tile_expert;
  int tile_m;
  int topk;
  int a_by_row;              // A row index = row (FC2) instead of the pair's token (FC1)
  Seg seg[4];
  int nseg;
  const float* pair_w;       // PAIR / TOKEN weights (NULL = 1)
  const void* add;           // ADD
  float beta, lbeta;
  // MX operands: e8m0 scales of A (row-major [*, Kd/32]) and of the packed weights
  const uint8_t* a_scale;
  uint32_t a_scale_bytes;
  const uint8_t* w_scale;
  uint8_t* out_scale;        // SITU_MX: [rows_cap, n_out/32]
  // split-K of the dense tiled GEMM: ksplit workgroups per tile each sum one slice of K
  // into `part` ([ksplit][M][sum of the segments' n_total] fp32); a reduce kernel adds
  // the slices in order and applies the epilogues. ksplit <= 1: no split.
  float* part;
  int ksplit;
};

// live_tiles: expected number of 16-row tiles that hold rows (sizes the split-K factor).
hipError_t launch_stream_gemm(StreamGemm g, Elt elt, int live_tiles, hipStream_t stream);
// LDS-tiled bf16 GEMM: 128-row tiles (dense rows, or grouped tiles with tile_m == 128); Kd % 128 == 0.
hipError_t launch_tiled_gemm(StreamGemm g, hipStream_t stream);
// Split-K factor the tiled kernel would use for dense g (1: none) and the fp32 workspace
// bytes it then needs.
int tiled_splitk(const StreamGemm& g);
size_t tiled_splitk_bytes(const StreamGemm& g, int ksplit);
// MXFP8 x packed MXFP4 (grouped mode, one segment: SITU_MX or PAIR / TOKEN); Kd % 512 == 0.
hipError_t launch_stream_gemm_mx(StreamGemm g, int live_tiles, hipStream_t stream);

hipError_t launch_route(int T, int E, int K, const float* logits, const float* bias, float rsf, int renorm,
                        int32_t* ids, float* weights, hipStream_t stream);

size_t permute_workspace_bytes(int npairs, int E);
hipError_t launch_permute(int npairs, int E, int tile_m, int max_tiles, const int32_t* ids, int32_t* counts,
                          int32_t* offsets, int32_t* tile_offsets, int32_t* row_to_pair, int32_t* tile_expert,
                          int32_t* pair_to_row, void* workspace, hipStream_t stream);

hipError_t launch_route_renormalize(int T, int E, int K, const float* logits, int32_t* ids, float* weights,
                                    hipStream_t stream);
hipError_t launch_route_grouped(int T, int E, int K, int n_group, int topk_group, const float* logits,
                                const float* bias, float rsf, int renorm, int32_t* ids, float* weights,
                                hipStream_t stream);

// Routing then permutation (one workgroup when route_permute_fusable(T, K)).
bool route_permute_fusable(int T, int K);
hipError_t launch_route_permute(int T, int E, int K, const float* logits, const float* bias, float rsf,
                                int renorm, int32_t* ids, float* weights, int tile_m, int max_tiles,
                                int32_t* counts, int32_t* offsets, int32_t* tile_offsets, int32_t* row_to_pair,
                                int32_t* tile_expert, int32_t* pair_to_row, void* workspace, hipStream_t stream);

hipError_t launch_situ_masked(int E, int T_max, int d, Elt elt, const void* in, const int32_t* counts,
                              float beta, float lbeta, void* out, hipStream_t stream);
hipError_t launch_quant_mxfp8(int rows, int cols, Elt elt, const void* in, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream);
hipError_t launch_combine(int T, int K, int N, const float* ws, Elt out_elt, void* out, hipStream_t stream);
hipError_t launch_pack_weights(int batch, int N, int Kd, int esize, const void* src, void* dst, hipStream_t stream);
hipError_t launch_pack_mxfp4(int batch, int N, int Kd, const void* codes_src, const void* scales_src, void* codes_dst,
                             void* scales_dst, hipStream_t stream);
// Combine (fixed k order) into fp32 z and RMSNorm of z into out, one workgroup per token.
hipError_t launch_combine_norm(int T, int K, int L, const float* ws, float* z, const void* gamma, float eps, Elt elt,
                               void* out, hipStream_t stream);
hipError_t launch_rmsnorm(int T, int L, const float* z, const void* gamma, float eps, Elt elt, void* out,
                          hipStream_t stream);

}  // namespace lmoe
