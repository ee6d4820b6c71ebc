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
