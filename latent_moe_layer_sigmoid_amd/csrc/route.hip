// Single-group sigmoid top-k routing for gfx950 (vLLM PR 50088, "What's in it",
// commit 1: with n_group == topk_group == 1 the grouped rule reduces to the K best of
// every expert, result k in lane k; commit 4: sigmoid scores, selection bias, routed scaling
// factor, FP32 logits).
//
// One wavefront (64 lanes) per token. Lane l owns experts l, l+64, l+128, ... and keeps
// their keys as a list sorted in descending order (a Batcher odd-even merge network in
// registers, on keys encoded as positive doubles so that each compare-exchange is an fp64
// max and min). A key is (order-preserving bits of sigmoid(logit) + bias, ~expert): the
// larger key wins and equal scores resolve to the lower expert index. Each of the K
// rounds takes the wave maximum of the lanes' list heads in two 32-bit passes (score
// bits, then ~expert among the lanes holding the top score) with DPP row shifts and row
// broadcasts, so a round costs a dozen VALU operations and no LDS traffic; the winning
// lane pops its head and lane k keeps round k's expert. Weights are then formed from the
// unbiased scores of the K winners (lanes 0..K-1), renormalized and scaled.
#include <math.h>

#include "kernels.h"
#include "route_dev.h"

namespace lmoe {

template <int KPL, int NP>
__global__ __launch_bounds__(256) void route_kernel(int T, int E, int K, const float* __restrict__ logits,
                                                    const float* __restrict__ bias, float rsf, int renorm,
                                                    int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int e;
  float w;
  route_token<KPL, NP>(t, E, K, logits, bias, rsf, renorm, &e, &w);
  if (lane < K) {
    ids[(size_t)t * K + lane] = e;
    weights[(size_t)t * K + lane] = w;
  }
}

// "Renormalize" routing: one wavefront per token, keys are the bf16-cast logits.
template <int KPL, int NP>
__global__ __launch_bounds__(256) void route_renorm_kernel(int T, int E, int K, const float* __restrict__ logits,
                                                           int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int e;
  float w;
  route_token<KPL, NP, 1>(t, E, K, logits, nullptr, 1.0f, 1, &e, &w);
  if (lane < K) {
    ids[(size_t)t * K + lane] = e;
    weights[(size_t)t * K + lane] = w;
  }
}

// Grouped top-k: one wavefront per token. The bias-corrected scores go to this wavefront's
// LDS row; the lanes of group g find its two largest scores (the group score is their fp32
// sum); lane g ranks group g against the other groups (ties -> lower group) and a ballot gives the
// wave-uniform mask of the topk_group kept groups; then the single-group routine runs
// with the other groups' experts left out.
template <int KPL, int NP>
__global__ __launch_bounds__(256) void route_grouped_kernel(int T, int E, int K, int n_group, int topk_group,
                                                            const float* __restrict__ logits,
                                                            const float* __restrict__ bias, float rsf, int renorm,
                                                            int32_t* __restrict__ ids, float* __restrict__ weights) {
  extern __shared__ float s_kap[];         // [4][E + 64]: scores, then group scores
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;                      // whole wavefronts; no workgroup barrier below
  float* kap = s_kap + wv * (E + 64);
  float* gsc = kap + E;
  const float* row = logits + (size_t)t * E;
  {   // every logit and bias requested before the first score is stored
    float lg[KPL], bs[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int e = min(lane + 64 * j, E - 1);
      lg[j] = row[e];
      bs[j] = bias ? bias[e] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int e = lane + 64 * j;
      if (e < E) kap[e] = score_of(lg[j]) + bs[j];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int gs = E / n_group;
  // lpg lanes per group (a power of two): each takes every lpg-th score of its group, then
  // the partial (largest, second largest) pairs merge by butterfly inside the group. The
  // two largest values of a group do not depend on the order they are met in.
  int lpg = 1;
  while (lpg * 2 * n_group <= 64) lpg *= 2;
  const int g = lane / lpg, sub = lane % lpg;
  float t1 = -INFINITY, t2 = -INFINITY;
  if (g < n_group) {
#pragma unroll 8
    for (int i = sub; i < gs; i += lpg) {
      const float v = kap[g * gs + i];
      if (v > t1) {
        t2 = t1;
        t1 = v;
      } else if (v > t2) {
        t2 = v;
      }
    }
  }
  for (int off = 1; off < lpg; off <<= 1) {
    const float u1 = __shfl_xor(t1, off, WAVE), u2 = __shfl_xor(t2, off, WAVE);
    const float n2 = fmaxf(fminf(t1, u1), fmaxf(t2, u2));
    t1 = fmaxf(t1, u1);
    t2 = n2;
  }
  if (g < n_group && sub == 0) gsc[g] = gs > 1 ? t1 + t2 : t1;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  bool keep = false;
  if (lane < n_group) {
    const float mine = gsc[lane];
    int rank = 0;
    for (int h = 0; h < n_group; ++h) {
      const float o = gsc[h];
      rank += (o > mine || (o == mine && h < lane)) ? 1 : 0;
    }
    keep = rank < topk_group;
  }
  const uint64_t keep_mask = __ballot(keep);
  int e;
  float w;
  route_token<KPL, NP, 0>(t, E, K, logits, bias, rsf, renorm, &e, &w, gs, keep_mask);
  if (lane < K) {
    ids[(size_t)t * K + lane] = e;
    weights[(size_t)t * K + lane] = w;
  }
}

hipError_t launch_route_renormalize(int T, int E, int K, const float* logits, int32_t* ids, float* weights,
                                    hipStream_t stream) {
  dim3 grid((T + 3) / 4), block(256);
#define LMOE_ROUTE_RN(KPL, NP) \
  hipLaunchKernelGGL((route_renorm_kernel<KPL, NP>), grid, block, 0, stream, T, E, K, logits, ids, weights)
  if (E <= 64) LMOE_ROUTE_RN(1, 1);
  else if (E <= 128) LMOE_ROUTE_RN(2, 2);
  else if (E <= 256) LMOE_ROUTE_RN(4, 4);
  else if (E <= 512) LMOE_ROUTE_RN(8, 8);
  else if (E <= 896) LMOE_ROUTE_RN(14, 16);
  else LMOE_ROUTE_RN(16, 16);
#undef LMOE_ROUTE_RN
  return hipGetLastError();
}

hipError_t launch_route_grouped(int T, int E, int K, int n_group, int topk_group, const float* logits,
                                const float* bias, float rsf, int renorm, int32_t* ids, float* weights,
                                hipStream_t stream) {
  dim3 grid((T + 3) / 4), block(256);
  const size_t lds = (size_t)4 * (E + 64) * sizeof(float);
#define LMOE_ROUTE_G(KPL, NP)                                                                                 \
  hipLaunchKernelGGL((route_grouped_kernel<KPL, NP>), grid, block, lds, stream, T, E, K, n_group, topk_group, \
                     logits, bias, rsf, renorm, ids, weights)
  if (E <= 64) LMOE_ROUTE_G(1, 1);
  else if (E <= 128) LMOE_ROUTE_G(2, 2);
  else if (E <= 256) LMOE_ROUTE_G(4, 4);
  else if (E <= 512) LMOE_ROUTE_G(8, 8);
  else if (E <= 896) LMOE_ROUTE_G(14, 16);
  else LMOE_ROUTE_G(16, 16);
#undef LMOE_ROUTE_G
  return hipGetLastError();
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
