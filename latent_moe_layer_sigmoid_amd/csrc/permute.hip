// Stable expert-sorted permutation of the (token, slot) pairs for gfx950: the per-expert
// row map that the expert GEMMs and the weighted combine consume, padded to the GEMM's row
// tile (TensorRT-LLM PR 20541, "Commit 1: routing as its own op").
//
// Pairs p = t*K + k are cut into blocks of 1024. Counts are order-free (LDS atomics);
// ranks inside an expert must follow pair order, so each block ranks its pairs with
// wave ballots: lanes holding the same expert are matched bit by bit over the expert id
// (one ballot per bit), the rank inside the wave is the popcount of matching lower
// lanes, and the per-wave counts in LDS give the offset of each earlier wave.
//   1 block  : one fused kernel (count, scan, rank, scatter).
//   >1 blocks: count per block (and -1 into every row of row_to_pair) -> one-block scan:
//              per expert, each block's exclusive prefix over the blocks (in place) and the
//              totals, then the expert scan -> per block: its base in each expert, rank +
//              scatter.
// Threads of a workgroup share data through LDS only, so its barriers order LDS alone (the
// global outputs are read by later launches).
// Decode-sized batches (T <= 16 tokens, T*K <= 1024 pairs) can also run routing and the
// permutation as one workgroup: wavefront t routes token t (TensorRT-LLM PR 20541,
// "Commit 1": routing produces the expert GEMMs' row map), the ids stay in LDS
// and the single-block permutation follows after a barrier.
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "route_dev.h"

namespace lmoe {

constexpr int PB = 1024;          // pairs per block (one per thread)
constexpr int PW = PB / WAVE;     // waves per block

// Mask of the lanes whose expert equals this lane's (inactive lanes pass e = -1).
LMOE_DEV uint64_t match_lanes(int e, int nbits) {
  uint64_t m = __ballot(e >= 0);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = e >= 0 && ((e >> b) & 1);
    const uint64_t on = __ballot(bit);
    m &= bit ? on : ~on;
  }
  return e >= 0 ? m : 0;
}

LMOE_DEV int lanes_below(uint64_t m, int lane) {
  return __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
}

// Inclusive sum of x over the lanes of the wavefront (lane i gets lanes 0..i): row shifts
// 1, 2, 4, 8 scan each row of 16 lanes (lanes shifted in from outside the row read 0), then
// row broadcasts of lanes 15 and 31 add the earlier rows' totals. The sums wrap modulo 2^32
// (unsigned), so a packed pair of 16-bit sums may carry into bit 31.
template <int CTRL, int ROW_MASK, bool BOUND_CTRL>
LMOE_DEV uint32_t dpp_add(uint32_t x) {
  return x + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, BOUND_CTRL);
}
LMOE_DEV uint32_t wave_inclusive_sum(uint32_t x) {
  x = dpp_add<0x111, 0xF, true>(x);    // row_shr:1
  x = dpp_add<0x112, 0xF, true>(x);    // row_shr:2
  x = dpp_add<0x114, 0xF, true>(x);    // row_shr:4
  x = dpp_add<0x118, 0xF, true>(x);    // row_shr:8
  x = dpp_add<0x142, 0xA, false>(x);   // row_bcast:15 -> rows 1, 3
  x = dpp_add<0x143, 0xC, false>(x);   // row_bcast:31 -> rows 2, 3
  return x;
}

// Block-wide exclusive scan of v over PB threads (modulo 2^32); returns the prefix and sets
// *total.
LMOE_DEV uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_sum(v);
  if (lane == 63) s_wave[w] = x;
  lds_sync();
  if (w == 0) {
    const uint32_t s = wave_inclusive_sum(lane < PW ? s_wave[lane] : 0u);
    if (lane < PW) s_wave[PW + lane] = s;   // inclusive per-wave totals
  }
  lds_sync();
  const uint32_t before = (w ? s_wave[PW + w - 1] : 0u) + x - v;
  *total = s_wave[2 * PW - 1];
  lds_sync();
  return before;
}

// Scan of counts over experts (each thread owns a contiguous range of experts), writing
// offsets, tile_offsets, the tile -> expert map and, with fill_pad, -1 into the pad rows.
// s_cnt holds counts[E]. While every padded row index fits in 16 bits, the two sums
// (pairs and padded rows) share one scan as the halves of a 32-bit value.
LMOE_DEV void scan_experts(const int* s_cnt, int E, int tile_m, int max_tiles, int32_t* counts,
                           int32_t* offsets, int32_t* tile_offsets, int32_t* row_to_pair,
                           int32_t* tile_expert, int* s_scratch, int* s_tile_off, bool fill_pad = true) {
  const int per = (E + PB - 1) / PB;
  const int e0 = threadIdx.x * per, e1 = min(E, e0 + per);
  const int tsh = __builtin_ctz(tile_m);   // tile_m is a power of two
  const int tmask = tile_m - 1;
  int c_sum = 0, p_sum = 0;
  for (int e = e0; e < e1; ++e) {
    const int c = s_cnt[e];
    c_sum += c;
    p_sum += (c + tmask) & ~tmask;
  }
  int c_tot, p_tot, c_pre, p_pre;
  uint32_t* s_u = reinterpret_cast<uint32_t*>(s_scratch);
  if ((long)max_tiles * tile_m < 65536) {
    // both sums stay below 2^16: the padded-row sum in the high half (it may reach bit 31,
    // so the word is decoded unsigned), the pair sum in the low half
    uint32_t tot;
    const uint32_t pre = block_exclusive_scan(((uint32_t)p_sum << 16) | (uint32_t)c_sum, s_u, &tot);
    c_pre = (int)(pre & 0xFFFFu);
    p_pre = (int)(pre >> 16);
    c_tot = (int)(tot & 0xFFFFu);
    p_tot = (int)(tot >> 16);
  } else {
    uint32_t ct, pt;
    c_pre = (int)block_exclusive_scan((uint32_t)c_sum, s_u, &ct);
    p_pre = (int)block_exclusive_scan((uint32_t)p_sum, s_u, &pt);
    c_tot = (int)ct;
    p_tot = (int)pt;
  }
  for (int e = e0; e < e1; ++e) {
    const int c = s_cnt[e];
    const int pc = (c + tmask) & ~tmask;
    counts[e] = c;
    offsets[e] = c_pre;
    tile_offsets[e] = p_pre;
    if (s_tile_off) s_tile_off[e] = p_pre;
    if (fill_pad)
      for (int r = p_pre + c; r < p_pre + pc; ++r) row_to_pair[r] = -1;
    for (int tt = p_pre >> tsh; tt < (p_pre + pc) >> tsh; ++tt) tile_expert[tt] = e;
    c_pre += c;
    p_pre += pc;
  }
  if (threadIdx.x == 0) {
    offsets[E] = c_tot;
    tile_offsets[E] = p_tot;
  }
  for (int tt = (p_tot >> tsh) + threadIdx.x; tt < max_tiles; tt += PB) tile_expert[tt] = -1;
}

// Rank the block's pairs inside their experts (pair order) and scatter them.
// base(e): first row for this block's pairs of expert e.
template <typename BaseFn>
LMOE_DEV void rank_scatter(const int32_t* ids, int npairs, int E, int nbits, int block0,
                           unsigned short* s_wcnt, BaseFn base, int32_t* row_to_pair,
                           int32_t* pair_to_row) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int p = block0 + threadIdx.x;
  const int e = p < npairs ? ids[p] : -1;
  const int rows = min(PW, (npairs - block0 + WAVE - 1) / WAVE);   // waves of this block holding pairs
  for (int i = threadIdx.x; i < rows * E; i += PB) s_wcnt[i] = 0;
  lds_sync();
  const uint64_t m = match_lanes(e, nbits);
  const int r_in_wave = lanes_below(m, lane);
  if (e >= 0 && r_in_wave == 0) s_wcnt[w * E + e] = (unsigned short)__popcll(m);
  lds_sync();
  if (e >= 0) {
    int r = r_in_wave;
    for (int w2 = 0; w2 < w; ++w2) r += s_wcnt[w2 * E + e];
    const int row = base(e) + r;
    row_to_pair[row] = p;
    pair_to_row[p] = row;
  }
}

LMOE_DEV int id_bits(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

// ---- single block: everything in one launch ---------------------------------------------
__global__ __launch_bounds__(PB) void permute_fused_kernel(int npairs, int E, int tile_m, int max_tiles,
                                                           const int32_t* __restrict__ ids, int32_t* counts,
                                                           int32_t* offsets, int32_t* tile_offsets,
                                                           int32_t* row_to_pair, int32_t* tile_expert,
                                                           int32_t* pair_to_row) {
  extern __shared__ int smem[];
  int* s_cnt = smem;                      // [E]
  int* s_toff = s_cnt + E;                // [E]
  int* s_scr = s_toff + E;                // [2 * PW]
  unsigned short* s_wcnt = (unsigned short*)(s_scr + 2 * PW);   // [PW * E]
  for (int e = threadIdx.x; e < E; e += PB) s_cnt[e] = 0;
  lds_sync();
  if ((int)threadIdx.x < npairs) atomicAdd(&s_cnt[ids[threadIdx.x]], 1);
  lds_sync();
  scan_experts(s_cnt, E, tile_m, max_tiles, counts, offsets, tile_offsets, row_to_pair, tile_expert,
               s_scr, s_toff);
  lds_sync();
  rank_scatter(ids, npairs, E, id_bits(E), 0, s_wcnt, [&](int e) { return s_toff[e]; }, row_to_pair,
               pair_to_row);
}

// ---- routing + permutation in one workgroup ------------------------------------------------
template <int KPL, int NP>
__global__ __launch_bounds__(PB) void route_permute_kernel(int T, int E, int K, const float* __restrict__ logits,
                                                           const float* __restrict__ bias, float rsf, int renorm,
                                                           int32_t* ids, float* weights, int tile_m, int max_tiles,
                                                           int32_t* counts, int32_t* offsets, int32_t* tile_offsets,
                                                           int32_t* row_to_pair, int32_t* tile_expert,
                                                           int32_t* pair_to_row) {
  extern __shared__ int smem[];
  const int npairs = T * K;
  int* s_cnt = smem;                      // [E]
  int* s_toff = s_cnt + E;                // [E]
  int* s_scr = s_toff + E;                // [2 * PW]
  int* s_ids = s_scr + 2 * PW;            // [T * K]
  unsigned short* s_wcnt = (unsigned short*)(s_ids + npairs);   // [PW * E]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += PB) s_cnt[e] = 0;
  if (w < T) {                            // whole wavefronts: token w
    int e;
    float wt;
    route_token<KPL, NP>(w, E, K, logits, bias, rsf, renorm, &e, &wt);
    if (lane < K) {
      ids[(size_t)w * K + lane] = e;
      weights[(size_t)w * K + lane] = wt;
      s_ids[w * K + lane] = e;
    }
  }
  lds_sync();
  if ((int)threadIdx.x < npairs) atomicAdd(&s_cnt[s_ids[threadIdx.x]], 1);
  lds_sync();
  scan_experts(s_cnt, E, tile_m, max_tiles, counts, offsets, tile_offsets, row_to_pair, tile_expert,
               s_scr, s_toff);
  lds_sync();
  rank_scatter(s_ids, npairs, E, id_bits(E), 0, s_wcnt, [&](int e) { return s_toff[e]; }, row_to_pair,
               pair_to_row);
}

bool route_permute_fusable(int T, int K) { return T <= PW && T * K <= PB; }

hipError_t launch_route_permute(int T, int E, int K, const float* logits, const float* bias, float rsf,
                                int renorm, int32_t* ids, float* weights, int tile_m, int max_tiles,
                                int32_t* counts, int32_t* offsets, int32_t* tile_offsets, int32_t* row_to_pair,
                                int32_t* tile_expert, int32_t* pair_to_row, void* workspace,
                                hipStream_t stream) {
  if (!route_permute_fusable(T, K)) {
    hipError_t err = launch_route(T, E, K, logits, bias, rsf, renorm, ids, weights, stream);
    if (err != hipSuccess) return err;
    return launch_permute(T * K, E, tile_m, max_tiles, ids, counts, offsets, tile_offsets, row_to_pair,
                          tile_expert, pair_to_row, workspace, stream);
  }
  const size_t sm = (size_t)(2 * E + 2 * PW + T * K) * sizeof(int) + (size_t)PW * E * sizeof(unsigned short);
#define LMOE_RP(KPL, NP)                                                                                    \
  hipLaunchKernelGGL((route_permute_kernel<KPL, NP>), dim3(1), dim3(PB), sm, stream, T, E, K, logits, bias, \
                     rsf, renorm, ids, weights, tile_m, max_tiles, counts, offsets, tile_offsets, row_to_pair, \
                     tile_expert, pair_to_row)
  if (E <= 64) LMOE_RP(1, 1);
  else if (E <= 128) LMOE_RP(2, 2);
  else if (E <= 256) LMOE_RP(4, 4);
  else if (E <= 512) LMOE_RP(8, 8);
  else if (E <= 896) LMOE_RP(14, 16);
  else LMOE_RP(16, 16);
#undef LMOE_RP
  return hipGetLastError();
}

// ---- several blocks ------------------------------------------------------------------------
__global__ __launch_bounds__(PB) void permute_count_kernel(int npairs, int E, const int32_t* __restrict__ ids,
                                                           int32_t* __restrict__ block_counts,
                                                           int32_t* __restrict__ row_to_pair, int rows_cap) {
  extern __shared__ int s_cnt[];
  // every row starts as padding; the scatter kernel (a later launch) writes the pairs
  for (int r = blockIdx.x * PB + threadIdx.x; r < rows_cap; r += gridDim.x * PB) row_to_pair[r] = -1;
  for (int e = threadIdx.x; e < E; e += PB) s_cnt[e] = 0;
  lds_sync();
  const int p = blockIdx.x * PB + threadIdx.x;
  if (p < npairs) atomicAdd(&s_cnt[ids[p]], 1);
  lds_sync();
  for (int e = threadIdx.x; e < E; e += PB) block_counts[(size_t)blockIdx.x * E + e] = s_cnt[e];
}

// One block: for each expert, the running sum over the blocks of its block counts,
// written back in place as each block's exclusive prefix (the pairs of that expert in the
// blocks before it; 32 counts requested together), the total kept in LDS; then the expert
// scan (the pad rows are already -1).
__global__ __launch_bounds__(PB) void permute_scan_kernel(int nblk, int E, int tile_m, int max_tiles,
                                                          int32_t* __restrict__ block_counts, int32_t* counts,
                                                          int32_t* offsets, int32_t* tile_offsets,
                                                          int32_t* row_to_pair, int32_t* tile_expert) {
  extern __shared__ int smem[];
  int* s_cnt = smem;          // [E]
  int* s_scr = s_cnt + E;     // [2 * PW]
  for (int e = threadIdx.x; e < E; e += PB) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += 32) {
      int c[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) c[j] = b0 + j < nblk ? block_counts[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (b0 + j < nblk) block_counts[(size_t)(b0 + j) * E + e] = run;
        run += c[j];
      }
    }
    s_cnt[e] = run;
  }
  lds_sync();
  scan_experts(s_cnt, E, tile_m, max_tiles, counts, offsets, tile_offsets, row_to_pair, tile_expert,
               s_scr, nullptr, false);
}

// block_counts holds, per block and expert, the pairs of that expert in earlier blocks.
__global__ __launch_bounds__(PB) void permute_scatter_kernel(int npairs, int E, const int32_t* __restrict__ ids,
                                                             const int32_t* __restrict__ block_before,
                                                             const int32_t* __restrict__ tile_offsets,
                                                             int32_t* row_to_pair, int32_t* pair_to_row) {
  extern __shared__ int s_base[];                                           // [E]
  unsigned short* s_wcnt = reinterpret_cast<unsigned short*>(s_base + E);   // [PW * E]
  // first row of this block's pairs in each expert
  for (int e = threadIdx.x; e < E; e += PB)
    s_base[e] = tile_offsets[e] + block_before[(size_t)blockIdx.x * E + e];
  lds_sync();
  rank_scatter(ids, npairs, E, id_bits(E), blockIdx.x * PB, s_wcnt, [&](int e) { return s_base[e]; },
               row_to_pair, pair_to_row);
}

size_t permute_workspace_bytes(int npairs, int E) {
  const int nblk = (npairs + PB - 1) / PB;
  return nblk <= 1 ? 0 : (size_t)nblk * E * sizeof(int32_t);
}

hipError_t launch_permute(int npairs, int E, int tile_m, int max_tiles, const int32_t* ids, int32_t* counts,
                          int32_t* offsets, int32_t* tile_offsets, int32_t* row_to_pair,
                          int32_t* tile_expert, int32_t* pair_to_row, void* workspace, hipStream_t stream) {
  const int nblk = (npairs + PB - 1) / PB;
  if (nblk <= 1) {
    const size_t sm = (size_t)(2 * E + 2 * PW) * sizeof(int) + (size_t)PW * E * sizeof(unsigned short);
    hipLaunchKernelGGL(permute_fused_kernel, dim3(1), dim3(PB), sm, stream, npairs, E, tile_m, max_tiles, ids,
                       counts, offsets, tile_offsets, row_to_pair, tile_expert, pair_to_row);
    return hipGetLastError();
  }
  int32_t* block_counts = (int32_t*)workspace;
  hipLaunchKernelGGL(permute_count_kernel, dim3(nblk), dim3(PB), (size_t)E * sizeof(int), stream, npairs, E,
                     ids, block_counts, row_to_pair, max_tiles * tile_m);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(PB), (size_t)(E + 2 * PW) * sizeof(int), stream, nblk, E,
                     tile_m, max_tiles, block_counts, counts, offsets, tile_offsets, row_to_pair, tile_expert);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(PB),
                     (size_t)E * sizeof(int) + (size_t)PW * E * sizeof(unsigned short), stream, npairs, E, ids,
                     block_counts, tile_offsets, row_to_pair, pair_to_row);
  return hipGetLastError();
}

// ---- permutation without a caller workspace ------------------------------------------------
// The per-block expert counts of the multi-block path live in a fixed device array of this
// library (one copy per GPU, held until the process ends). Its name is only a host-side
// stand-in for the device address, so the address each device gives it is looked up once
// per device and kept.
static __device__ __align__(256) int32_t scratch[PERMUTE_SCRATCH_BYTES / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t permute_scratch(void** ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `dev` current
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace lmoe
