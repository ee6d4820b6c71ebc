// Argument types of the GEMM kernels of liblmoe (internal): element types, epilogues,
// output segments and the launch description shared by the weight-streaming, tiled and
// MX kernels.
#pragma once
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
  // every weight row is read by a single 16-row tile of this launch (dense M <= 16, or
  // grouped with at most 16 tokens): the stream kernel then loads weights non-temporally
  int weights_once;
};

}  // namespace lmoe
