// LDS-tiled MFMA GEMM for gfx950 (bf16 in, fp32 accumulate) for the token-heavy calls:
// the prefill-sized projections of the hidden input, the tail, and the grouped expert
// FC1 / FC2 over tiles of 128 expert rows.
//
// Workgroup tile 128 rows x 128 weight rows (a SituGLU block takes 64 gate rows and the
// matching 64 up rows), K stage of 128, 256 threads = 4 wavefronts in a 2 x 2 grid, each
// owning 64 x 64 outputs as 4 x 4 v_mfma_f32_16x16x32_bf16 tiles. Both operands reach LDS
// by direct buffer-to-LDS loads (buffer_load_dwordx4 ... lds), arranged in the packed MFMA
// order the weights already have in HBM: for each 16-row group and 32-wide K slice q, a
// 1 KB block holding lane l = 16g + r's 16 bytes (row r, K 8g .. 8g + 7) at 16 l. Every
// MFMA operand is then one conflict-free 1 KB ds_read_b128, and the weights are copied
// block by block. Two LDS stages (2 x 64 KB): stage c + 1 is requested before stage c is
// computed. Workgroups are remapped so that consecutive tiles share an XCD (and its L2).
// Epilogues as in the weight-streaming kernel: plain store, SituGLU (vLLM PR 50088,
// commit 2), weighted per-pair store for the combine (TensorRT-LLM PR 20541, "Commit 1":
// finalize), and the in-place add of the up projection (vLLM latent_moe_runner page,
// _shard_up_proj_tail).
#include "common.h"
#include "kernels.h"

namespace lmoe {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int TILE_M = 128;
constexpr int STAGE = 65536;      // bytes per LDS stage: A 32 KB + B 32 KB
constexpr int B_OFF = 32768;

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector-memory operations of
// this wave are outstanding; expcnt and lgkmcnt unconstrained.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

LMOE_DEV void to_lds(rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

LMOE_DEV void store_out(Elt elt, void* base, size_t idx, float v) {
  if (elt == Elt::F32)
    reinterpret_cast<float*>(base)[idx] = v;
  else
    reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16(v);
}

__global__ __launch_bounds__(256) void tiled_gemm_kernel(const StreamGemm g, int blocks_total, int nch) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  constexpr int NACC = 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m = lane & 15, g4 = lane >> 4;

  // consecutive logical tiles on one XCD (workgroups are dealt to the 8 XCDs in turn)
  const int G = gridDim.x;
  const int bid = (G & 7) == 0 ? (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int mt = bid / blocks_total;
  const int nb_all = bid - mt * blocks_total;
  const int row0 = mt * TILE_M;
  if (row0 >= g.M) return;

  int s = 0;
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (i < g.nseg && nb_all >= g.seg[i].block0) s = i;
  const Seg sg = g.seg[s];
  const int nb = nb_all - sg.block0;
  const bool situ = sg.epi == Epi::SITU;
  const bool grouped = g.row_to_pair != nullptr;
  int e = 0;
  if (grouped) {
    e = g.tile_expert[row0 / g.tile_m];
    if (e < 0) return;
  }

  // ---- rows this wave loads into LDS (groups 2*wave, 2*wave+1) and their byte offsets
  int arow[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = row0 + 16 * (2 * wave + h) + m;
    if (grouped) {
      int p = g.row_to_pair[row];
      const bool real = p >= 0;
      if (!real) p = g.row_to_pair[row0];               // the tile's first row is always a real pair
      arow[h] = g.a_by_row ? (real ? row : row0) : p / g.topk;
    } else {
      arow[h] = min(row, g.M - 1);
    }
  }
  const rsrc_t a_rs = make_rsrc(g.a, g.a_bytes);
  uint32_t a_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) a_off[h] = (uint32_t)arow[h] * (uint32_t)(g.lda * 2) + g4 * 16;

  // ---- weight row groups this wave loads (LDS groups 2*wave, 2*wave+1)
  const uint32_t w_bytes = (uint32_t)sg.n_total * (uint32_t)(g.Kd * 2);
  const rsrc_t w_rs = make_rsrc(reinterpret_cast<const char*>(sg.w) + (size_t)e * w_bytes, w_bytes);
  uint32_t b_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int jj = 2 * wave + h;
    const int n16 = situ ? (jj < 4 ? nb * 4 + jj : sg.n_out / 16 + nb * 4 + (jj - 4)) : nb * 8 + jj;
    b_off[h] = (uint32_t)n16 * (uint32_t)nch * 4096u + lane * 16;   // past the matrix: zeros
  }

  auto issue = [&](int c, int st) {
    char* base = smem + st * STAGE;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        to_lds(a_rs, base + ((2 * wave + h) * 4 + q) * 1024, a_off[h], (uint32_t)c * 256u + q * 64u);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        to_lds(w_rs, base + B_OFF + ((2 * wave + h) * 4 + q) * 1024, b_off[h], (uint32_t)c * 4096u + q * 1024u);
  };

  floatx4 acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

  int bgrp[4];   // LDS weight groups of this wave's four column tiles
#pragma unroll
  for (int j = 0; j < 4; ++j) bgrp[j] = situ ? (j < 2 ? 2 * wn + j : 4 + 2 * wn + (j - 2)) : 4 * wn + j;

  auto compute = [&](int st) {
    const char* base = smem + st * STAGE;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(base + ((4 * wm + i) * 4 + q) * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(base + B_OFF + (bgrp[j] * 4 + q) * 1024 + lane * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i * 4 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i * 4 + j], 0, 0, 0);
    }
  };

  issue(0, 0);
  for (int c = 0; c < nch; ++c) {
    if (c + 1 < nch) {
      issue(c + 1, (c + 1) & 1);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(16));   // this wave's stage-c requests have landed
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __syncthreads();                                 // ... and every other wave's
    compute(c & 1);
    __syncthreads();                                 // stage c & 1 is free for stage c + 2
  }

  // ---- epilogue: tile (i, j): rows row0 + 64 wm + 16 i + 4 g4 + rr, column lane m
  const float inv_b = 1.0f / g.beta;
  const float inv_lb = g.lbeta > 0.0f ? 1.0f / g.lbeta : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = row0 + 64 * wm + 16 * i + 4 * g4 + rr;
      int pair = row;
      if (grouped) {
        pair = g.row_to_pair[row];
        if (pair < 0) continue;
      } else if (row >= g.M) {
        continue;
      }
      if (situ) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = 64 * nb + 32 * wn + 16 * j + m;
          if (col >= sg.n_out) continue;
          const float v = situ_f(acc[i * 4 + j][rr], acc[i * 4 + j + 2][rr], g.beta, inv_b, g.lbeta, inv_lb);
          store_out(sg.out_elt, sg.out, (size_t)row * sg.ldo + col, v);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = 128 * nb + 64 * wn + 16 * j + m;
          if (col >= sg.n_out) continue;
          float v = acc[i * 4 + j][rr];
          if (sg.epi == Epi::STORE) {
            store_out(sg.out_elt, sg.out, (size_t)row * sg.ldo + col, v);
          } else if (sg.epi == Epi::PAIR) {
            const float wgt = g.pair_w ? g.pair_w[pair] : 1.0f;
            reinterpret_cast<float*>(sg.out)[(size_t)pair * sg.ldo + col] = wgt * v;
          } else if (sg.epi == Epi::TOKEN) {
            const float wgt = g.pair_w ? g.pair_w[pair] : 1.0f;
            store_out(sg.out_elt, sg.out, (size_t)(pair / g.topk) * sg.ldo + col, wgt * v);
          } else if (sg.epi == Epi::ADD) {
            const size_t idx = (size_t)row * sg.ldo + col;
            const float add = g.add ? (sg.out_elt == Elt::F32 ? reinterpret_cast<const float*>(g.add)[idx]
                                                               : bf16_to_f32(reinterpret_cast<const uint16_t*>(g.add)[idx]))
                                    : 0.0f;
            store_out(sg.out_elt, sg.out, idx, add + v);
          }
        }
      }
    }
}

hipError_t launch_tiled_gemm(StreamGemm g, hipStream_t stream) {
  const int nch = g.Kd / 128;
  int b0 = 0;
  for (int i = 0; i < g.nseg; ++i) {
    const int per = g.seg[i].epi == Epi::SITU ? 64 : 128;
    g.seg[i].blocks = (g.seg[i].n_out + per - 1) / per;
    g.seg[i].block0 = b0;
    b0 += g.seg[i].blocks;
  }
  const int m_tiles = (g.M + TILE_M - 1) / TILE_M;
  hipLaunchKernelGGL(tiled_gemm_kernel, dim3((unsigned)(m_tiles * b0)), dim3(256), 0, stream, g, b0, nch);
  return hipGetLastError();
}

}  // namespace lmoe
