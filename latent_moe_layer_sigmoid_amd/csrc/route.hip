// Single-group sigmoid top-k routing for gfx950 (vLLM PR 50088, "What's in it",
// commit 1: with n_group == topk_group == 1 the grouped top-k is a plain top-k over all
// experts, result k in lane k; commit 4: sigmoid scores, selection bias, routed scaling
// factor, FP32 logits).
//
// One wavefront (64 lanes) per token. Lane l owns experts l, l+64, l+128, ... and keeps
// their keys as a list sorted in descending order (a Batcher odd-even merge network in
// registers). A key is (order-preserving bits of sigmoid(logit) + bias, ~expert): the
// larger key wins and equal scores resolve to the lower expert index. Each of the K
// rounds takes the wave maximum of the lanes' list heads in two 32-bit passes (score
// bits, then ~expert among the lanes holding the top score) with DPP row shifts and row
// broadcasts, so a round costs a dozen VALU operations and no LDS traffic; the winning
// lane pops its head and lane k keeps round k's expert. Weights are then formed from the
// unbiased scores of the K winners (lanes 0..K-1), renormalized and scaled.
#include "common.h"
#include "kernels.h"

namespace lmoe {

LMOE_DEV uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Maximum of x over the 64 lanes, returned as a wave-uniform value.
// Row shifts 1, 2, 4, 8 leave each row's maximum in its lane 15; two row broadcasts
// carry it to lane 63. Lanes reading outside their row see 0, the identity here.
LMOE_DEV uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true));   // row_shr:1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true));   // row_shr:2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true));   // row_shr:4
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true));   // row_shr:8
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

LMOE_DEV void cas_desc(uint64_t& a, uint64_t& b) {
  const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
  a = hi;
  b = lo;
}

// Batcher's odd-even merge sort of N (a power of two) keys, descending; fully unrolled.
template <int N>
LMOE_DEV void sort_desc(uint64_t* k) {
#pragma unroll
  for (int p = 1; p < N; p <<= 1)
#pragma unroll
    for (int q = p; q >= 1; q >>= 1)
#pragma unroll
      for (int j = q % p; j + q < N; j += 2 * q)
#pragma unroll
        for (int i = 0; i < q; ++i)
          if (i + j + q < N && (i + j) / (2 * p) == (i + j + q) / (2 * p)) cas_desc(k[i + j], k[i + j + q]);
}

LMOE_DEV float score_of(float logit) { return __builtin_amdgcn_rcpf(1.0f + __expf(-logit)); }

template <int KPL, int NP>   // keys per lane, padded to the power of two NP
__global__ __launch_bounds__(256) void route_kernel(int T, int E, int K, const float* __restrict__ logits,
                                                    const float* __restrict__ bias, float rsf, int renorm,
                                                    int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;

  // issue every load before the first use (clamped, in-bounds indices), then build keys
  float lg[KPL], bs[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int e = min(lane + 64 * j, E - 1);
    lg[j] = row[e];
    bs[j] = bias ? bias[e] : 0.0f;
  }
  uint64_t key[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int e = lane + 64 * j;
    key[j] = 0;   // below every real key; never selected since K <= E
    if (j < KPL && e < E) {
      const float kap = score_of(lg[j]) + bs[j];
      key[j] = ((uint64_t)orderable(kap) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
  }
  sort_desc<NP>(key);

  uint32_t my_lo = 0;
  for (int k = 0; k < K; ++k) {
    const uint32_t hh = (uint32_t)(key[0] >> 32), ll = (uint32_t)key[0];
    const uint32_t mh = wave_max_u32(hh);
    const uint32_t ml = wave_max_u32(hh == mh ? ll : 0u);
    if (hh == mh && ll == ml) {   // the unique winning lane pops its head
#pragma unroll
      for (int j = 0; j + 1 < NP; ++j) key[j] = key[j + 1];
      key[NP - 1] = 0;
    }
    if (lane == k) my_lo = ml;
  }
  int e = 0;
  float s = 0.0f;
  if (lane < K) {
    e = (int)(0xFFFFFFFFu - my_lo);
    s = score_of(row[e]);   // same expression as at selection time
  }
  float sum = s;            // butterfly: every lane ends with the same total
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) sum += __shfl_xor(sum, off, WAVE);
  if (lane < K) {
    ids[(size_t)t * K + lane] = e;
    weights[(size_t)t * K + lane] = renorm ? rsf * s / sum : rsf * s;
  }
}

hipError_t launch_route(int T, int E, int K, const float* logits, const float* bias, float rsf, int renorm,
                        int32_t* ids, float* weights, hipStream_t stream) {
  dim3 grid((T + 3) / 4), block(256);
#define LMOE_ROUTE(KPL, NP)                                                                         \
  hipLaunchKernelGGL((route_kernel<KPL, NP>), grid, block, 0, stream, T, E, K, logits, bias, rsf, \
                     renorm, ids, weights)
  if (E <= 64) LMOE_ROUTE(1, 1);
  else if (E <= 128) LMOE_ROUTE(2, 2);
  else if (E <= 256) LMOE_ROUTE(4, 4);
  else if (E <= 512) LMOE_ROUTE(8, 8);
  else if (E <= 896) LMOE_ROUTE(14, 16);
  else LMOE_ROUTE(16, 16);
#undef LMOE_ROUTE
  return hipGetLastError();
}

}  // namespace lmoe
