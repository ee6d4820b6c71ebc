// Host-side launchers of the gfx950 kernels (internal to liblmoe).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gemm_types.h"

namespace lmoe {

// live_tiles: expected number of 16-row tiles that hold rows (sizes the split-K factor);
// target_waves: wavefronts the launch aims for (0: the default of 2048).
hipError_t launch_stream_gemm(StreamGemm g, Elt elt, int live_tiles, hipStream_t stream, long target_waves = 0);
// LDS-tiled bf16 GEMM: 128-row tiles (dense rows, or grouped tiles with tile_m == 128); Kd % 128 == 0.
hipError_t launch_tiled_gemm(StreamGemm g, hipStream_t stream);
bool tiled_dual_ok(const StreamGemm& g);
// Split-K factor the tiled kernel would use for dense g (1: none) and the fp32 workspace
// bytes it then needs.
int tiled_splitk(const StreamGemm& g);
size_t tiled_splitk_bytes(const StreamGemm& g, int ksplit);
// Output columns of a dense M-row launch that fill whole rounds of the CUs, when the rest
// is small enough to run with split K (n_out: no split).
int tiled_round_cols(int M, int n_out);
// MXFP8 x packed MXFP4 (grouped mode, one segment: SITU_MX or PAIR / TOKEN); Kd % 512 == 0.
hipError_t launch_stream_gemm_mx(StreamGemm g, int live_tiles, hipStream_t stream);

hipError_t launch_route(int T, int E, int K, const float* logits, const float* bias, float rsf, int renorm,
                        int32_t* ids, float* weights, hipStream_t stream);

size_t permute_workspace_bytes(int npairs, int E);
// Device scratch of the permutation when the caller brings no workspace: this device's
// copy of a fixed array of PERMUTE_SCRATCH_BYTES (looked up once per device).
constexpr size_t PERMUTE_SCRATCH_BYTES = size_t(1) << 20;
hipError_t permute_scratch(void** ptr);
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
