/* lmoe.h -- C ABI of the latent-MoE layer forward for AMD Instinct MI355X (gfx950).
 *
 * The layer (one GPU, full share of the work):
 *   router GEMM -> single-group sigmoid top-k routing -> latent down projection
 *   -> expert-sorted permutation -> grouped FC1 + SituGLU -> grouped FC2 + weighted
 *   combine -> latent RMSNorm -> up projection with the shared-expert add.
 *
 * Sources cited below:
 *   [P1] vLLM pull request 50088, "[MoE] Latent-MoE runner, fused MoE tail, SituGLU
 *        activation and single-group top-k routing", section "What's in it", commits 1-7.
 *   [P2] TensorRT-LLM pull request 20541 (Kimi K3 MoE decode, router stream),
 *        sections "Description" and "Commit 1: routing as its own op".
 *   [P3] vLLM API page vllm.models.kimi_k3.amd.latent_moe_runner, ROCmLatentMoERunner
 *        (_fused_forward, _shard_up_proj_tail, enable_quantized_routed_input).
 *   [OCP-MX] OCP Microscaling Formats (MX) v1.0 (E4M3, E2M1, E8M0, blocks of 32).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers, densely packed. Activations are row-major.
 *     Weights have the logical shape [out, in] (the nn.Linear layout that [P3]
 *     _shard_up_proj_tail multiplies by weight.t()) and are passed to the compute calls
 *     in the packed layout written by lmoe_pack_weights (an MFMA-operand order in which
 *     every wave-wide load reads 1 KB of contiguous HBM).
 *   - The caller owns every buffer and the stream. A call validates its arguments on
 *     the host, enqueues kernels on `stream` and returns; results are valid once the
 *     stream reaches the call ([P2] "Commit 1": routing is an op on the current stream
 *     writing caller-allocated outputs). The library never allocates device memory,
 *     never synchronizes and keeps no per-call state, so calls from several host
 *     threads are safe on distinct buffers.
 *   - Errors are returned, never thrown; an invalid call enqueues nothing. Contract
 *     violations that only the device can see (an expert id >= E inside topk_ids,
 *     counts that do not match the ids) are undefined behaviour.
 *   - T == 0 (or rows == 0) is a successful no-op that touches no HIP API.
 *   - dtype pairs supported: activations and weights both LMOE_F32 or both LMOE_BF16
 *     (fp32 accumulate); for the expert GEMMs also activations LMOE_MXFP8_E4M3 with
 *     weights LMOE_MXFP4_E2M1 (scaled MFMA, fp32 accumulate).
 */
#ifndef LMOE_H
#define LMOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LMOE_ABI_VERSION 1

typedef enum {
  LMOE_OK = 0,
  LMOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, beta <= 0, mismatched dtypes, ... */
  LMOE_ERR_UNSUPPORTED = 2, /* no kernel for this shape / dtype combination */
  LMOE_ERR_WORKSPACE = 3,   /* workspace or capacity too small ([P2] "Commit 1": the runner validates the workspace) */
  LMOE_ERR_HIP = 4          /* a HIP launch error was reported */
} lmoe_status;

typedef enum {
  LMOE_F32 = 0,
  LMOE_BF16 = 1,
  LMOE_MXFP8_E4M3 = 2, /* one byte per element + one E8M0 scale byte per 32 elements */
  LMOE_MXFP4_E2M1 = 3  /* two elements per byte (element 2i low nibble) + one E8M0 byte per 32 */
} lmoe_dtype;

int lmoe_abi_version(void);
const char* lmoe_status_string(lmoe_status s);

/* Weight packing: the HBM layout of every weight argument below. src holds `batch`
 * row-major matrices [N, Kd]; dst (same byte size, not overlapping src) receives them
 * packed. Let KCH = 256 / esize (128 bf16 or 64 fp32 elements = 256 bytes of a row). For
 * 16-row group n16 and K chunk c, the 4 KB block at byte (n16 * (Kd / KCH) + c) * 4096
 * of a matrix holds, at byte q*1024 + g*256 + r*16 + i*esize (q, g < 4; r < 16;
 * i < 16 / esize), the element W[16*n16 + r][c*KCH + q*KCH/4 + g*KCH/16 + i].
 * Lane l = 16g + r of a wavefront reading 16 bytes at q*1024 + 16l thus receives the
 * B operand of one MFMA (column r, k-group g). dtype F32 or BF16; N % 16 == 0,
 * Kd % KCH == 0, else LMOE_ERR_UNSUPPORTED. */
lmoe_status lmoe_pack_weights(int batch, int N, int Kd, lmoe_dtype dtype, const void* src, void* dst,
                              hipStream_t stream);

/* MXFP4 weight packing for the MX expert GEMMs. src: `batch` matrices [N, Kd] as codes
 * [N, Kd/2] (two E2M1 per byte, element 2i in the low nibble) and E8M0 scales [N, Kd/32];
 * dst: same sizes, packed. For 16-row group n16 and 512-wide K stage s (nst = Kd / 512):
 * the codes' 4 KB block at byte (n16*nst + s)*4096 holds at byte q*1024 + g*256 + r*16 + j
 * the source code byte (s*512 + q*128 + g*32)/2 + j of row 16*n16 + r (j < 16); the
 * scales' 256-byte block at (n16*nst + s)*256 holds at byte (16g + r)*4 + q the scale of
 * K block s*16 + q*4 + g of that row. Lane l = 16g + r then holds one 32-element MX block
 * per scaled MFMA. N % 16 == 0 and Kd % 512 == 0, else LMOE_ERR_UNSUPPORTED. */
lmoe_status lmoe_pack_mxfp4_weights(int batch, int N, int Kd, const uint8_t* codes_src, const uint8_t* scales_src,
                                    uint8_t* codes_dst, uint8_t* scales_dst, hipStream_t stream);

/* Dense projection (router GEMM, latent down projection) y[M,N] = x[M,Kd] @ w[N,Kd]^T with fp32 accumulation.
 * Used for the router GEMM (y LMOE_F32: [P1] commit 4, DeepSeekV3 routing takes FP32
 * logits; [P2] "Description": the router GEMM runs first) and the latent down projection
 * ([P2] "Description"; [P3] _fused_forward: routed input transform on hidden).
 * x_dtype == w_dtype in {F32, BF16}; y_dtype in {F32, BF16}. Kd % 128 == 0 (BF16) or
 * Kd % 64 == 0 (F32), N % 16 == 0, else LMOE_ERR_UNSUPPORTED. */
lmoe_status lmoe_linear(int M, int N, int Kd, lmoe_dtype x_dtype, const void* x,
                        lmoe_dtype w_dtype, const void* w, lmoe_dtype y_dtype, void* y,
                        hipStream_t stream);

/* Several projections of one input in one launch -- up to four of them:
 *   y_i = x @ w_i^T                                    (situ == NULL or situ[i] == 0), or
 *   y_i = SituGLU(x @ w_i^T) with w_i of 2*N[i] rows   (situ[i] != 0; gate rows first)
 * for i < n_proj <= 4. The decode-time projections of the hidden input -- the router GEMM
 * (fp32 logits), the latent down projection and the shared expert's FC1 with its SituGLU
 * ([P2] "Commit 2": router GEMM, shared experts and latent down projection all start
 * from the hidden states; [P3] _fused_forward: the shared experts take the untransformed
 * hidden) -- read x once per column block and share one launch. Per projection: N[i]
 * output columns (N[i] % 16 == 0), packed weights w[i], output y[i] [M, N[i]] of
 * y_dtype[i] (F32 or BF16). beta / linear_beta as in lmoe_fc1_situ (checked only when
 * some situ[i] != 0). x_dtype F32 or BF16 (also the weights' dtype); Kd as lmoe_linear. */
lmoe_status lmoe_linear_multi(int M, int Kd, lmoe_dtype x_dtype, const void* x, int n_proj, const int* N,
                              const void* const* w, const lmoe_dtype* y_dtype, void* const* y, const int* situ,
                              float beta, float linear_beta, hipStream_t stream);

/* lmoe_linear_multi with a caller-provided fp32 workspace for split-K: when M is large
 * enough for the LDS-tiled kernel (BF16, M >= 256) but its 128 x 512 tiles would leave
 * CUs idle, each tile's K range is cut into slices computed by separate workgroups into
 * `workspace`, and a second kernel adds the slices in fixed order and applies the
 * epilogues (results are reproducible; they may differ in the last bits from the
 * unsplit call). lmoe_linear_multi_workspace_bytes returns the bytes this call needs for
 * the same shapes (0: no split, workspace unused). workspace NULL: no split; non-NULL but
 * smaller than needed: LMOE_ERR_WORKSPACE. */
size_t lmoe_linear_multi_workspace_bytes(int M, int Kd, lmoe_dtype x_dtype, int n_proj, const int* N,
                                         const int* situ);
lmoe_status lmoe_linear_multi_ws(int M, int Kd, lmoe_dtype x_dtype, const void* x, int n_proj, const int* N,
                                 const void* const* w, const lmoe_dtype* y_dtype, void* const* y, const int* situ,
                                 float beta, float linear_beta, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Single-group DeepSeekV3 top-k routing ([P1] commit 1: with one group the
 * grouped rule reduces to choosing the K best of every expert, result k held in lane k; [P1]
 * commit 4: sigmoid scores, selection bias, routed scaling factor, FP32 logits).
 *   s = sigmoid(logits[t, :]);  selection key = s + bias (bias may be NULL = 0);
 *   topk_ids[t, k]  = expert with the k-th largest key (ties -> lower expert index);
 *   topk_weights[t, k] = rsf * s[id] / sum_j s[id_j]   (renormalize != 0)
 *                      = rsf * s[id]                   (renormalize == 0).
 * logits fp32 [T,E]; bias fp32 [E]; topk_ids int32 [T,K]; topk_weights fp32 [T,K].
 * 1 <= K <= min(E, 64) (the sorting-network bound of [P1] commit 1); E <= 1024. */
lmoe_status lmoe_route(int T, int E, int K, const float* logits, const float* bias,
                       float routed_scaling_factor, int renormalize,
                       int32_t* topk_ids, float* topk_weights, hipStream_t stream);

/* Grouped top-k routing, the general case of lmoe_route ([P1] commit 1: n_group ==
 * topk_group == 1 is the degenerate case of the grouped kernels; [P1] commit 4: sigmoid +
 * grouped top-k with the selection bias, group counts and routed scaling factor). The
 * pages give no formula; this follows DeepSeek-V3's rule: with key = sigmoid(logit) +
 * bias (fp32), the E experts form n_group contiguous groups of E / n_group; a group's
 * score is the fp32 sum of its two largest keys (its only key for groups of one); the
 * topk_group groups with the highest scores are kept (ties -> lower group index);
 * topk_ids are the K largest keys among the kept groups' experts (ties -> lower expert
 * index, slot order descending) and topk_weights are formed as in lmoe_route.
 * n_group == 1 (or topk_group == n_group) gives exactly lmoe_route. Requirements:
 * 1 <= n_group <= 64, E % n_group == 0, 1 <= topk_group <= n_group,
 * K <= topk_group * (E / n_group), plus those of lmoe_route. */
lmoe_status lmoe_route_grouped(int T, int E, int K, int n_group, int topk_group, const float* logits,
                               const float* bias, float routed_scaling_factor, int renormalize,
                               int32_t* topk_ids, float* topk_weights, hipStream_t stream);

/* "Renormalize" routing ([P1] commit 4: on this path the logits are cast to BF16 and no
 * bias, group counts or routed scaling factor are used; [P2] "Test Coverage": Renormalize
 * next to the DeepSeekV3 method). The fp32 logits are rounded to bf16 (nearest even);
 * topk_ids[t, k] = expert with the k-th largest bf16 logit (ties -> lower expert index);
 * topk_weights[t, k] = softmax of the K selected bf16 logits (fp32). 1 <= K <= min(E, 64),
 * E <= 1024. */
lmoe_status lmoe_route_renormalize(int T, int E, int K, const float* logits, int32_t* topk_ids,
                                   float* topk_weights, hipStream_t stream);

/* Stable expert-sorted permutation of the T*K (token, slot) pairs, pair p = t*K + k
 * (the per-expert row map that the expert GEMMs and the
 * weighted combine consume, padded to the expert GEMM's row tile; [P2] "Commit 1"). Outputs (all int32, caller-allocated):
 *   expert_counts[E]       pairs routed to each expert;
 *   expert_offsets[E+1]    exclusive prefix sum of the counts;
 *   tile_offsets[E+1]      exclusive prefix sum of counts rounded up to tile_m;
 *   row_to_pair[rows_cap]  for rows r < tile_offsets[E]: the pair in row r, -1 on pad
 *                          rows; pairs of one expert are in ascending pair order;
 *   tile_expert[rows_cap / tile_m]  expert of each tile of tile_m rows, -1 past the end;
 *   pair_to_row[T*K]       inverse of row_to_pair.
 * tile_m in {16, 32, 64, 128, 256}. rows_cap >= lmoe_permute_rows_cap(T, E, K, tile_m) and
 * a multiple of tile_m, else LMOE_ERR_WORKSPACE. workspace: device scratch of at least
 * lmoe_permute_workspace_bytes(T, E, K) bytes (NULL allowed when that is 0). */
size_t lmoe_permute_workspace_bytes(int T, int E, int K);
int lmoe_permute_rows_cap(int T, int E, int K, int tile_m);
lmoe_status lmoe_permute(int T, int E, int K, int tile_m, const int32_t* topk_ids,
                         int32_t* expert_counts, int32_t* expert_offsets, int32_t* tile_offsets,
                         int32_t* row_to_pair, int32_t* tile_expert, int32_t* pair_to_row,
                         int rows_cap, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* lmoe_permute for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments,
 * checks and results as lmoe_permute, minus the workspace. The per-block counts of
 * batches above 1024 pairs go to a fixed scratch array inside the library, one copy per
 * GPU, of lmoe_permute_noalloc_max_bytes() bytes (1 MiB), held until the process ends;
 * a call needing more than that (ceil(T*K / 1024) * E * 4 bytes, i.e. above about 292k
 * pairs at E = 896) returns LMOE_ERR_WORKSPACE and enqueues nothing. The call allocates
 * nothing; its first call on a device looks up that device's scratch address once.
 * `stream` must belong to the current device (else LMOE_ERR_INVALID_ARG). Every call on
 * one GPU shares that GPU's scratch: calls that may overlap in time on one GPU (on
 * different streams, or from several host threads) race and must be serialized by the
 * caller. The scratch needs no clearing: each call writes every count it reads. */
size_t lmoe_permute_noalloc_max_bytes(void);
lmoe_status lmoe_permute_noalloc(int T, int E, int K, int tile_m, const int32_t* topk_ids,
                                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* tile_offsets,
                                 int32_t* row_to_pair, int32_t* tile_expert, int32_t* pair_to_row,
                                 int rows_cap, hipStream_t stream);

/* Routing followed by the permutation, in one launch for decode-sized batches
 * (T <= 16 and T*K <= 1024: one workgroup routes each token with one wavefront, keeps the
 * ids on chip and builds the permutation from them; [P2] "Commit 1": the routing op
 * produces the row map the expert GEMMs use). Larger batches run lmoe_route then
 * lmoe_permute. Arguments, outputs, checks and error codes are exactly those of the two
 * calls (topk_ids and topk_weights are written as by lmoe_route; workspace as for
 * lmoe_permute); results are identical to the two calls made in sequence. */
lmoe_status lmoe_route_permute(int T, int E, int K, const float* logits, const float* bias,
                               float routed_scaling_factor, int renormalize,
                               int32_t* topk_ids, float* topk_weights, int tile_m,
                               int32_t* expert_counts, int32_t* expert_offsets, int32_t* tile_offsets,
                               int32_t* row_to_pair, int32_t* tile_expert, int32_t* pair_to_row,
                               int rows_cap, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* MXFP8 (E4M3) quantization along rows ([OCP-MX]; [P2] "Description": input
 * quantization before the MXE4M3 x MXE2M1 experts; [P1] commit 3: outside the fused
 * SiLU path, the activation output is quantized again afterwards). Per 32 consecutive elements:
 * exponent X = floor(log2 max|v|) - 8 clamped to [-127,127] (0 for an all-zero block);
 * code = E4M3(v / 2^X), nearest-even, saturating at 448, sign bit set for v < 0.
 * in [rows, cols] (F32 or BF16), codes u8 [rows, cols], scales u8 [rows, cols/32] = X+127.
 * cols % 32 == 0. */
lmoe_status lmoe_quant_mxfp8(int rows, int cols, lmoe_dtype in_dtype, const void* in,
                             uint8_t* codes, uint8_t* scales, hipStream_t stream);

/* Grouped FC1 with the SituGLU epilogue ([P1] commit 2: SituGLU,
 * fp32 accumulate, written straight to the output; [P1] commit 5: SituGLU acts on the
 * dequantized gate/up; [P3] enable_quantized_routed_input: gate and up not interleaved).
 *   For every row r of a tile with expert e = tile_expert[r / tile_m] >= 0 and pair
 *   p = row_to_pair[r] >= 0, with token t = p / K:
 *     h = a[t, :] @ w1[e]^T           (w1 [E, 2d, in_dim]; h[:d] gate, h[d:] up)
 *     act[r, j] = SituGLU(h[j], h[d+j]) = beta*tanh(g/beta)*sigmoid(g)
 *                 * (linear_beta > 0 ? linear_beta*tanh(u/linear_beta) : u)
 *   Rows with p < 0 (padding) and rows of tiles with expert -1 are never written.
 * Dense mode (the shared expert): row_to_pair == NULL and tile_expert == NULL, E == 1,
 * K == 1: row r = token r for r < T.
 * beta must be finite and > 0 ([P1] commit 3: beta is required); linear_beta <= 0 means
 * unset (passes up through). tile_m must be the tile the permutation was built with.
 * a_dtype/w_dtype: F32/F32 or BF16/BF16 with act_dtype == a_dtype; or MXFP8_E4M3 /
 * MXFP4_E2M1 (grouped mode only; a_scale [T, in_dim/32] row-major, w1 and w1_scale
 * packed by lmoe_pack_mxfp4_weights, in_dim % 512 == 0, d % 32 == 0) with act_dtype
 * MXFP8_E4M3: SituGLU in fp32 on the dequantized accumulators, then each 32 consecutive
 * outputs requantized as lmoe_quant_mxfp8 does (act codes [rows_cap, d], act_scale
 * [rows_cap, d/32]). */
lmoe_status lmoe_fc1_situ(int T, int E, int K, int in_dim, int d, int tile_m,
                          lmoe_dtype a_dtype, const void* a, const uint8_t* a_scale,
                          const int32_t* row_to_pair, const int32_t* tile_expert,
                          lmoe_dtype w_dtype, const void* w1, const uint8_t* w1_scale,
                          float beta, float linear_beta,
                          lmoe_dtype act_dtype, void* act, uint8_t* act_scale,
                          int rows_cap, hipStream_t stream);

/* lmoe_fc1_situ with a bound on the launch's width, for a call that runs on a second
 * stream beside latency-bound work on the first ([P2] "Commit 2": the shared experts on
 * their own stream, overlapping the router and the routed experts). The weight-streaming
 * launch (bf16 / fp32 below 256 tokens) then aims for about max_waves wavefronts instead
 * of 2048 (rounded to its shape: column blocks x K splits), so it takes a smaller share of
 * the HBM bandwidth and finishes later; max_waves == 0 keeps the default, and the tiled
 * and MX launches ignore it. Arguments and checks are those of lmoe_fc1_situ; so are the
 * results, except that with fewer wavefronts K is split over fewer partial sums, so the
 * fp32 accumulation adds in another order (same error bound; bit for bit only when
 * max_waves == 0). max_waves < 0 gives LMOE_ERR_INVALID_ARG. */
lmoe_status lmoe_fc1_situ_capped(int T, int E, int K, int in_dim, int d, int tile_m,
                                 lmoe_dtype a_dtype, const void* a, const uint8_t* a_scale,
                                 const int32_t* row_to_pair, const int32_t* tile_expert,
                                 lmoe_dtype w_dtype, const void* w1, const uint8_t* w1_scale,
                                 float beta, float linear_beta,
                                 lmoe_dtype act_dtype, void* act, uint8_t* act_scale,
                                 int rows_cap, int max_waves, hipStream_t stream);

/* Grouped FC2 with the weighted combine ([P2] "Commit 1": the combine uses the
 * routing row map; [P3] enable_quantized_routed_input: router weights are applied
 * after the experts, not on their input).
 *   y_r = act[r, :] @ w2[e]^T (w2 [E, out_dim, d]) for every valid row r, then
 *   out[t, :] = sum_{k=0..K-1} topk_weights[t, k] * y_{pair_to_row(t*K+k)}   (k ascending),
 *   `out` [T, out_dim] is overwritten. topk_weights NULL means weight 1.
 * With K > 1 the per-pair products go through `workspace` (>= lmoe_fc2_workspace_bytes
 * bytes) and are summed in fixed k order, so the result is bitwise reproducible.
 * Dense mode as in lmoe_fc1_situ (shared expert: E == 1, K == 1).
 * act_dtype/w_dtype: F32/F32, BF16/BF16, or MXFP8_E4M3/MXFP4_E2M1 (grouped mode only;
 * act_scale [rows_cap, d/32] row-major; w2, w2_scale packed by lmoe_pack_mxfp4_weights;
 * d % 512 == 0, out_dim % 64 == 0). out_dtype F32 or BF16. */
size_t lmoe_fc2_workspace_bytes(int T, int K, int out_dim);
lmoe_status lmoe_fc2_combine(int T, int E, int K, int d, int out_dim, int tile_m,
                             lmoe_dtype act_dtype, const void* act, const uint8_t* act_scale,
                             const int32_t* row_to_pair, const int32_t* tile_expert,
                             lmoe_dtype w_dtype, const void* w2, const uint8_t* w2_scale,
                             const float* topk_weights, lmoe_dtype out_dtype, void* out,
                             int rows_cap, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* FC2 + combine + latent RMSNorm, the FC2 half of the layer ending in the normalized
 * latent that the up projection reads: exactly lmoe_fc2_combine with out_dtype F32 and
 * out = z, followed by the RMSNorm of lmoe_tail (norm_out = z / sqrt(mean(z^2) + eps) *
 * gamma, in fp32; gamma [out_dim] and norm_out [T, out_dim] in norm_dtype, F32 or BF16).
 * With K > 1 one kernel sums each token's K products (fixed k order) and normalizes the
 * sum, which it also stores in z; results are bit-identical to the two separate calls.
 * Pass latent = NULL to lmoe_tail / lmoe_tail_shared afterwards. Extra checks: eps >= 0
 * and finite, out_dim % 4 == 0, norm_out != NULL and != z (when T > 0). */
lmoe_status lmoe_fc2_combine_norm(int T, int E, int K, int d, int out_dim, int tile_m,
                                  lmoe_dtype act_dtype, const void* act, const uint8_t* act_scale,
                                  const int32_t* row_to_pair, const int32_t* tile_expert,
                                  lmoe_dtype w_dtype, const void* w2, const uint8_t* w2_scale,
                                  const float* topk_weights, float* z, int rows_cap,
                                  void* workspace, size_t workspace_bytes, const void* gamma, float eps,
                                  lmoe_dtype norm_dtype, void* norm_out, hipStream_t stream);

/* Latent tail ([P1] commit 7: the routed output is summed before the
 * output transform because it contains an RMSNorm; [P3] _shard_up_proj_tail: norm of
 * the reduced latent, then shared += latent @ up_proj^T in the GEMM's epilogue; [P1]
 * commit 6: the up projection folds in the shared-expert add).
 *   norm_out[t, :] = latent[t, :] / sqrt(mean(latent[t, :]^2) + eps) * gamma   (fp32 math)
 *   out[t, :]      = shared[t, :] + norm_out[t, :] @ w_up^T
 * latent fp32 [T, L]; gamma [L] in io_dtype (NULL = ones); w_up [H, L] in io_dtype;
 * shared, out [T, H] in io_dtype (shared NULL = no add; out may alias shared);
 * norm_out [T, L] in io_dtype (caller-owned, also returned). io_dtype F32 or BF16.
 * latent NULL: norm_out already holds the normalized latent (from lmoe_fc2_combine_norm)
 * and only the projection runs. eps >= 0. L % 128 == 0 (BF16) / 64 (F32), H % 16 == 0. */
lmoe_status lmoe_tail(int T, int L, int H, const float* latent, const void* gamma, float eps,
                      const void* w_up, const void* shared, lmoe_dtype io_dtype, void* out,
                      void* norm_out, hipStream_t stream);

/* The tail with the shared expert's FC2 folded into the up projection ([P3]
 * _shard_up_proj_tail: hidden += latent @ up_proj^T accumulated into the shared output;
 * [P1] commit 6: the up projection folds in the shared-expert add):
 *   norm_out = RMSNorm(latent; gamma, eps)                        (as lmoe_tail)
 *   T < 256 (or F32):  out[t, :] = round(round(shared_act[t, :] @ w_s2^T) + norm_out[t, :] @ w_up^T)
 *   T >= 256, BF16:    out[t, :] = round(shared_act[t, :] @ w_s2^T + norm_out[t, :] @ w_up^T)
 * where round() rounds to io_dtype. With few tokens the shared-expert output is rounded
 * exactly as if it had been stored, then added in fp32; with many, both products are
 * summed in one set of fp32 accumulators (one GEMM over both K ranges), which differs
 * from the first form by at most half a unit in the last place of the shared output
 * before the final rounding. shared_act [T, I] is the shared expert's
 * SituGLU activation, w_s2 [H, I] and w_up [H, L] packed weights. out must not alias
 * shared_act or norm_out. latent NULL: norm_out already holds the normalized latent.
 * L % 128 and I % 128 == 0 (BF16; 64 for F32), H % 16 == 0. */
lmoe_status lmoe_tail_shared(int T, int L, int H, int I, const float* latent, const void* gamma, float eps,
                             const void* w_up, const void* shared_act, const void* w_s2, lmoe_dtype io_dtype,
                             void* out, void* norm_out, hipStream_t stream);

/* lmoe_tail_shared with a caller-provided fp32 workspace for split-K: with T >= 256 (BF16)
 * and too few 128 x 512 output tiles to fill the CUs (for example T = 1024, H = 7168), the
 * K range of both phases together is cut into slices computed by separate workgroups into
 * `workspace`, and a second kernel adds the slices in fixed order and rounds (results are
 * reproducible; they may differ in the last bits from the unsplit call). When the tiles
 * make whole rounds of the 256 CUs plus at most half a round (for example T = 8192, H =
 * 7168: 896 tiles), the columns of the whole rounds are computed at full K, bit-identical
 * to the unsplit call, and only the remaining columns are split into slices.
 * lmoe_tail_shared_workspace_bytes returns the bytes needed for the same shapes (0: no
 * split, workspace unused). workspace NULL: no split; non-NULL but smaller than needed:
 * LMOE_ERR_WORKSPACE. Everything else as lmoe_tail_shared. */
size_t lmoe_tail_shared_workspace_bytes(int T, int L, int H, int I, lmoe_dtype io_dtype);
lmoe_status lmoe_tail_shared_ws(int T, int L, int H, int I, const float* latent, const void* gamma, float eps,
                                const void* w_up, const void* shared_act, const void* w_s2, lmoe_dtype io_dtype,
                                void* out, void* norm_out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Masked SituGLU over the batched [E, T_max, 2d] expert layout ([P1] commit 2:
 * the masked kernel takes each expert's valid row count and never touches rows past it).
 *   For e < E and r < clamp(expert_num_tokens[e], 0, T_max):
 *     out[e, r, j] = SituGLU(in[e, r, j], in[e, r, d + j]), fp32 math;
 *   every other element of `out` is left exactly as it was.
 * in [E, T_max, 2d], out [E, T_max, d], both `dtype` (F32 or BF16); d % 8 == 0. */
lmoe_status lmoe_situ_masked(int E, int T_max, int d, lmoe_dtype dtype, const void* in,
                             const int32_t* expert_num_tokens, float beta, float linear_beta,
                             void* out, hipStream_t stream);

/* ---- One layer step, and its HIP graph ----------------------------------------------
 * The calls above strung into one forward step of the layer, in the benchmark's schedule
 * ([P2] "Commit 2": the shared experts on their own stream, overlapping the router and
 * the routed experts, joined by an event before the routed reduction):
 *   main stream:   lmoe_linear_multi_ws (router GEMM -> fp32 logits, latent down
 *                  projection) -> routing + permutation (lmoe_route_permute; or
 *                  lmoe_route_grouped / lmoe_route_renormalize then lmoe_permute)
 *                  -> [MX: lmoe_quant_mxfp8] -> lmoe_fc1_situ -> lmoe_fc2_combine_norm
 *                  -> wait for the second stream -> lmoe_tail (shared FC2 on the second
 *                  stream) or lmoe_tail_shared_ws (shared FC2 folded into the tail);
 *   second stream: lmoe_fc1_situ_capped (the shared FC1, dense mode)
 *                  [-> lmoe_fc2_combine (the shared FC2) when it is not folded].
 * When the shared FC1's 128 x 512 tiles alone fill the CUs (ceil(T/128) * ceil(2I/512)
 * >= 256), the main stream also waits until the second stream has taken the fork, so the
 * shared FC1 starts first. With shared_stream == 0 everything runs on the caller's stream:
 * one lmoe_linear_multi_ws launch with the shared FC1 as its third projection, then the
 * routed path, then lmoe_tail_shared_ws. Results are those of the same calls made one by
 * one (bit for bit: the same launches in the same order).
 * [P2] measures its decode steps under CUDA graphs and checks graph runs bitwise against
 * eager ones ("Test Coverage"): lmoe_layer_capture records one step into a HIP graph held
 * by the layer object, and lmoe_layer_replay launches it.
 *
 * lmoe_layer_desc: shapes (T tokens, H hidden, L latent, E experts, K top-k, d expert
 * intermediate, I shared intermediate), the expert row tile tile_m, dtype (F32 or BF16:
 * activations, dense weights, gamma and outputs), mx_experts (0: W1 / W2 in dtype; 1:
 * MXFP4 expert weights with scales, the latent quantized to MXFP8), the routing method
 * (n_group / topk_group for LMOE_ROUTE_GROUPED; topk weights renormalized and scaled by
 * routed_scaling_factor as in lmoe_route), beta / linear_beta (SituGLU), eps (RMSNorm),
 * the packed weights (bias and gamma may be NULL), and the caller-owned device buffers
 * every call writes, with the sizes those calls require: logits [T,E] fp32, topk_ids /
 * topk_weights [T,K], the permutation outputs (rows_cap >= lmoe_permute_rows_cap and its
 * workspace), latent [T,L] (MX: latent_q [T,L] and latent_scales [T,L/32] too), act
 * [rows_cap,d] (MX: act_scales [rows_cap,d/32]), z [T,L] fp32 and fc2_ws
 * (lmoe_fc2_workspace_bytes), shared_act [T,I], shared_out [T,H] (needed only when the
 * shared FC2 is not folded), norm [T,L], out [T,H], and the optional split-K workspaces
 * of the front and tail launches (NULL: no split). shared_stream selects the schedule,
 * fold_shared_fc2 (-1: fold from 256 tokens in BF16, 0 / 1) the tail, side_waves the
 * bound passed to lmoe_fc1_situ_capped (0: its default), side_stream the second stream
 * (NULL: the layer creates its own; passing the stream the caller's other work already
 * uses keeps the process's streams from sharing hardware queues with the main stream,
 * which would serialize the two).
 *
 * lmoe_layer_create checks the description (pointers and buffer / workspace sizes, then
 * every call's shape and dtype rules by calling it with no tokens, which enqueues nothing)
 * and returns LMOE_ERR_INVALID_ARG / LMOE_ERR_UNSUPPORTED / LMOE_ERR_WORKSPACE as those
 * calls would. It copies the description and creates, on the current device, three events
 * and (shared_stream set, side_stream NULL) a second stream of default priority; the layer owns what it
 * creates and allocates no device buffer. lmoe_layer_forward enqueues one step reading x [T,H] on `stream` (which must
 * belong to the layer's device; the second stream joins and leaves it through events, so
 * the step is complete once `stream` reaches its end). Its calls were checked at
 * creation, so it fails only with LMOE_ERR_HIP (a launch error; the step may then be
 * partly enqueued) or LMOE_ERR_INVALID_ARG (another current device, x NULL).
 * lmoe_layer_capture records one step reading x into a HIP graph (stream capture of
 * `stream`, which must not be the legacy default stream; the graph replaces any earlier
 * one, and the HIP runtime allocates what it needs to instantiate it); nothing runs. The
 * graph reads x and writes the description's buffers at the addresses given, so a replay
 * uses x's contents at that time. lmoe_layer_replay launches the graph on `stream`
 * (LMOE_ERR_INVALID_ARG before a capture). A layer object is used by one host thread at a
 * time, and steps of one layer (eager or replayed) must not overlap in time: they share
 * the buffers and the second stream. lmoe_layer_destroy releases the graph, events and
 * stream (after the caller has waited for the layer's work); NULL is ignored. */
typedef enum { LMOE_ROUTE_SIGMOID = 0, LMOE_ROUTE_GROUPED = 1, LMOE_ROUTE_RENORMALIZE = 2 } lmoe_routing;

typedef struct lmoe_layer_desc {
  int T, H, L, E, K, d, I, tile_m;
  lmoe_dtype dtype;
  int mx_experts;
  lmoe_routing routing;
  int n_group, topk_group;
  float beta, linear_beta, routed_scaling_factor, eps;
  /* packed weights */
  const void* w_router;      /* [E, H] */
  const float* bias;         /* [E] fp32 selection bias, NULL = 0 */
  const void* w_down;        /* [L, H] */
  const void* w1;            /* [E, 2d, L] (MX: codes [E, 2d, L/2]) */
  const uint8_t* w1_scales;  /* MX: [E, 2d, L/32] */
  const void* w2;            /* [E, L, d] (MX: codes [E, L, d/2]) */
  const uint8_t* w2_scales;  /* MX: [E, L, d/32] */
  const void* w_s1;          /* [2I, H], gate rows first */
  const void* w_s2;          /* [H, I] */
  const void* gamma;         /* [L], NULL = ones */
  const void* w_up;          /* [H, L] */
  /* buffers */
  float* logits;
  int32_t* topk_ids;
  float* topk_weights;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* tile_offsets;
  int32_t* row_to_pair;
  int32_t* tile_expert;
  int32_t* pair_to_row;
  int rows_cap;
  void* perm_ws;
  size_t perm_ws_bytes;
  void* latent;
  uint8_t* latent_q;
  uint8_t* latent_scales;
  void* act;
  uint8_t* act_scales;
  float* z;
  void* fc2_ws;
  size_t fc2_ws_bytes;
  void* shared_act;
  void* shared_out;
  void* norm;
  void* out;
  void* front_ws;
  size_t front_ws_bytes;
  void* tail_ws;
  size_t tail_ws_bytes;
  /* schedule */
  int shared_stream;
  int fold_shared_fc2;
  int side_waves;
  hipStream_t side_stream;   /* the second stream (caller-owned, default priority); NULL: the layer creates one */
} lmoe_layer_desc;

typedef struct lmoe_layer lmoe_layer;

/* sizeof(lmoe_layer_desc) as this library was built (a binding checks its own layout). */
size_t lmoe_layer_desc_bytes(void);
lmoe_status lmoe_layer_create(const lmoe_layer_desc* desc, lmoe_layer** layer);
lmoe_status lmoe_layer_forward(lmoe_layer* layer, const void* x, hipStream_t stream);
lmoe_status lmoe_layer_capture(lmoe_layer* layer, const void* x, hipStream_t stream);
lmoe_status lmoe_layer_replay(lmoe_layer* layer, hipStream_t stream);
void lmoe_layer_destroy(lmoe_layer* layer);

#ifdef __cplusplus
}
#endif

#endif /* LMOE_H */
