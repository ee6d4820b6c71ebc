// Single-group sigmoid top-k routing for gfx950 (vLLM PR 50088, "What's in it",
// commit 1: with n_group == topk_group == 1 the grouped top-k is a plain top-k over all
// experts; commit 4: sigmoid scores, selection bias, routed scaling factor, FP32 logits).
//
// One wavefront (64 lanes) per token. Lane l holds experts l, l+64, l+128, ... as packed
// 64-bit keys (order-preserving bits of sigmoid(logit)+bias << 32 | ~expert), so one
// unsigned max picks the largest key and, among equal keys, the lower expert index.
// K rounds of a 6-step butterfly max extract the keys in descending order; round k's
// winner is kept by lane k, which then writes slot k (coalesced stores).
#include "common.h"
#include "kernels.h"

namespace lmoe {

LMOE_DEV uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int KPL>
__global__ __launch_bounds__(256) void route_kernel(int T, int E, int K, const float* __restrict__ logits,
                                                    const float* __restrict__ bias, float rsf, int renorm,
                                                    int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;

  uint64_t key[KPL];
  float score[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int e = lane + 64 * j;
    key[j] = 0;          // below every real key; never selected since K <= E
    score[j] = 0.0f;
    if (e < E) {
      const float s = 1.0f / (1.0f + expf(-row[e]));
      const float kap = s + (bias ? bias[e] : 0.0f);
      key[j] = ((uint64_t)orderable(kap) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
      score[j] = s;
    }
  }
  uint64_t best = key[0];
#pragma unroll
  for (int j = 1; j < KPL; ++j) best = key[j] > best ? key[j] : best;

  int my_id = 0;
  float my_s = 0.0f;
  for (int k = 0; k < K; ++k) {
    const uint64_t m = wave_max(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)m);
    float s_win = 0.0f;
    if (best == m) {   // exactly one lane: keys are unique through the index bits
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        if (key[j] == m) {
          s_win = score[j];
          key[j] = 0;
        }
      }
      best = key[0];
#pragma unroll
      for (int j = 1; j < KPL; ++j) best = key[j] > best ? key[j] : best;
    }
    const float s = __shfl(s_win, e & 63, WAVE);
    if (lane == k) {
      my_id = e;
      my_s = s;
    }
  }
  const float sum = wave_sum(lane < K ? my_s : 0.0f);
  if (lane < K) {
    const float w = renorm ? rsf * my_s / sum : rsf * my_s;
    ids[(size_t)t * K + lane] = my_id;
    weights[(size_t)t * K + lane] = w;
  }
}

hipError_t launch_route(int T, int E, int K, const float* logits, const float* bias, float rsf,
                        int renorm, int32_t* ids, float* weights, hipStream_t stream) {
  dim3 grid((T + 3) / 4), block(256);
#define LMOE_ROUTE(KPL)                                                                         \
  hipLaunchKernelGGL(route_kernel<KPL>, grid, block, 0, stream, T, E, K, logits, bias, rsf, \
                     renorm, ids, weights)
  if (E <= 64) LMOE_ROUTE(1);
  else if (E <= 128) LMOE_ROUTE(2);
  else if (E <= 256) LMOE_ROUTE(4);
  else if (E <= 512) LMOE_ROUTE(8);
  else if (E <= 896) LMOE_ROUTE(14);
  else LMOE_ROUTE(16);
#undef LMOE_ROUTE
  return hipGetLastError();
}

}  // namespace lmoe
