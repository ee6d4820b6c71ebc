// Weight-streaming MFMA GEMM for gfx950: y = A @ W^T over tiles of 16 rows.
//
// Built for the decode-sized calls of the layer, where every weight byte is read once
// and HBM bandwidth is the bound: the router GEMM and latent down projection, the
// routed experts' FC1 / FC2 (a handful of rows per touched expert), the shared expert
// and the up projection.
//
// One wavefront owns 16 rows x (16 * NT) output columns. Per 256-byte K-chunk, lane l
// (row / column l % 16, k-group l / 16) loads four 16-byte pieces of its activation row
// (row-major) and of each weight tile (packed MFMA layout: one contiguous 1 KB per load
// instruction, which streams HBM at full rate where row-major 64-byte pieces do not);
// piece q feeds one v_mfma_f32_16x16x32_bf16 (or four v_mfma_f32_16x16x4_f32) covering
// chunk elements [32q, 32q + 32) in the same order for A and B. The next chunk's loads
// are issued before the current chunk's MFMAs. Up to 8 wavefronts of a workgroup split the K range; their fp32
// partial tiles are summed in LDS in fixed wave order (deterministic), and wave 0 runs
// the fused epilogue: plain store, SituGLU (vLLM PR 50088, commit 2: gate = first d
// columns, up = last d), weighted per-pair store for the combine (TensorRT-LLM PR
// 20541, "Commit 1": finalize), or the shared-expert add of the up projection (vLLM API
// page latent_moe_runner, _shard_up_proj_tail: beta-add epilogue).
#include "common.h"
#include "kernels.h"

namespace lmoe {

struct Chunk {
  uint4 v[4];
};

// Operands are read with buffer loads: a wave-uniform resource (base address and byte
// size, range-checked by the hardware: reads past the end return zeros), a per-lane
// 32-bit byte offset that never changes, and the chunk offset in a scalar register, so
// the K loop carries no per-lane address arithmetic.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

LMOE_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Activation rows are row-major: lane l's share of a 256-byte chunk row is the four
// 16-byte pieces at 16 * (l / 16) + 64 * q, q = 0..3 (voff includes 16 * (l / 16)), so
// piece q holds k-slots [32q, 32q + 32) of the chunk in MFMA order.
LMOE_DEV Chunk load_chunk_a(rsrc_t r, uint32_t voff, uint32_t soff) {
  Chunk c;
  c.v[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  c.v[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 64, soff, 0));
  c.v[2] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 128, soff, 0));
  c.v[3] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 192, soff, 0));
  return c;
}

// Weights are in the packed layout (see lmoe_pack_weights): the 16 rows x 256 bytes of
// one (row group, chunk) form a 4 KB block whose piece q is the 1 KB at q * 1024 + 16 * l
// for lane l. Every load instruction reads 1 KB contiguous.
LMOE_DEV Chunk load_chunk_w(rsrc_t r, uint32_t voff, uint32_t soff) {
  Chunk c;
  c.v[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  c.v[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 1024, soff, 0));
  c.v[2] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 2048, soff, 0));
  c.v[3] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 3072, soff, 0));
  return c;
}

template <Elt ELT>
struct EltTraits;
template <>
struct EltTraits<Elt::BF16> {
  static constexpr int KCH = 128;   // elements per 256-byte chunk row
  static constexpr int BYTES = 2;
};
template <>
struct EltTraits<Elt::F32> {
  static constexpr int KCH = 64;
  static constexpr int BYTES = 4;
};

template <Elt ELT>
LMOE_DEV floatx4 mfma_chunk(const Chunk& a, const Chunk& b, floatx4 acc);

template <>
LMOE_DEV floatx4 mfma_chunk<Elt::BF16>(const Chunk& a, const Chunk& b, floatx4 acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v[q]),
                                                  __builtin_bit_cast(bf16x8_t, b.v[q]), acc, 0, 0, 0);
  }
  return acc;
}

template <>
LMOE_DEV floatx4 mfma_chunk<Elt::F32>(const Chunk& a, const Chunk& b, floatx4 acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float* fa = reinterpret_cast<const float*>(&a.v[q]);
    const float* fb = reinterpret_cast<const float*>(&b.v[q]);
#pragma unroll
    for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[c], fb[c], acc, 0, 0, 0);
  }
  return acc;
}

LMOE_DEV void store_elt(Elt elt, void* base, size_t idx, float v) {
  if (elt == Elt::F32)
    reinterpret_cast<float*>(base)[idx] = v;
  else
    reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16(v);
}

LMOE_DEV float load_elt(Elt elt, const void* base, size_t idx) {
  return elt == Elt::F32 ? reinterpret_cast<const float*>(base)[idx]
                         : bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}

template <Elt ELT, int NT>
__global__ __launch_bounds__(512) void stream_gemm_kernel(const StreamGemm g, int n_blocks, int kchunks) {
  using TR = EltTraits<ELT>;
  extern __shared__ float s_red[];   // [splits][NT][4][64] when splits > 1
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int splits = blockDim.x >> 6;
  const int mt = blockIdx.x / n_blocks;
  const int nb = blockIdx.x - mt * n_blocks;
  const int row0 = mt * 16;
  if (row0 >= g.M) return;
  const bool grouped = g.row_to_pair != nullptr;
  int e = 0;
  if (grouped) {
    e = g.tile_expert[row0 / g.tile_m];
    if (e < 0) return;
  }
  const int m = lane & 15;
  const int g4 = lane >> 4;

  // ---- A row of this lane
  int arow;
  if (grouped) {
    const int pair = g.row_to_pair[row0 + m];
    const uint64_t valid = __ballot(pair >= 0);
    if (valid == 0) return;                          // all-padding sub-tile (uniform per block)
    const int src = __ffsll((unsigned long long)valid) - 1;
    const int fill = __shfl(pair, src, WAVE);
    const int p = pair >= 0 ? pair : fill;
    const int r = pair >= 0 ? row0 + m : row0 + src;
    arow = g.a_by_row ? r : p / g.topk;
  } else {
    arow = min(row0 + m, g.M - 1);
  }
  const rsrc_t a_rs = make_rsrc(g.a, g.a_bytes);
  const uint32_t a_off = (uint32_t)arow * (uint32_t)(g.lda * TR::BYTES) + g4 * 16;

  // ---- weight rows (one per tile j)
  const int half = NT / 2;
  const uint32_t w_bytes = (uint32_t)g.n_total * (uint32_t)(g.Kd * TR::BYTES);   // one expert
  const rsrc_t w_rs = make_rsrc(reinterpret_cast<const char*>(g.w) + (size_t)e * w_bytes, w_bytes);
  uint32_t b_off[NT];   // start of tile j's row group in the packed layout, plus the lane's 16 bytes
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int n0;
    if (g.epi == Epi::SITU)
      n0 = (j < half) ? nb * half * 16 + j * 16 : g.d + nb * half * 16 + (j - half) * 16;
    else
      n0 = nb * NT * 16 + j * 16;
    b_off[j] = (uint32_t)(n0 / 16) * (uint32_t)kchunks * 4096u + lane * 16;
  }

  // ---- K range of this wave (wave-uniform)
  const int wu = __builtin_amdgcn_readfirstlane(wid);
  const int c0 = (int)((long)kchunks * wu / splits);
  const int c1 = (int)((long)kchunks * (wu + 1) / splits);
  constexpr int CB = TR::KCH * TR::BYTES;   // bytes per chunk row (256)

  floatx4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Ping-pong buffers: chunk c + 1 is requested before chunk c is consumed. The request
  // index is clamped to the wave's last chunk, so the final requests re-read a chunk that
  // is still cached instead of running past the range; they are never consumed.
  if (c0 < c1) {
    Chunk a0, a1, b0[NT], b1[NT];
    a0 = load_chunk_a(a_rs, a_off, (uint32_t)c0 * CB);
#pragma unroll
    for (int j = 0; j < NT; ++j) b0[j] = load_chunk_w(w_rs, b_off[j], (uint32_t)c0 * 4096u);
    int c = c0;
    // sched_barrier keeps the compiler from sinking the requests below the MFMAs that
    // consume the older buffer (which would serialize every chunk on memory latency).
    while (true) {
      const uint32_t o1 = (uint32_t)min(c + 1, c1 - 1);
      a1 = load_chunk_a(a_rs, a_off, o1 * CB);
#pragma unroll
      for (int j = 0; j < NT; ++j) b1[j] = load_chunk_w(w_rs, b_off[j], o1 * 4096u);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = mfma_chunk<ELT>(a0, b0[j], acc[j]);
      __builtin_amdgcn_sched_barrier(0);
      if (++c >= c1) break;
      const uint32_t o2 = (uint32_t)min(c + 1, c1 - 1);
      a0 = load_chunk_a(a_rs, a_off, o2 * CB);
#pragma unroll
      for (int j = 0; j < NT; ++j) b0[j] = load_chunk_w(w_rs, b_off[j], o2 * 4096u);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = mfma_chunk<ELT>(a1, b1[j], acc[j]);
      __builtin_amdgcn_sched_barrier(0);
      if (++c >= c1) break;
    }
  }

  // ---- split-K reduction in fixed wave order
  if (splits > 1) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_red[((wid * NT + j) * 4 + i) * 64 + lane] = acc[j][i];
    __syncthreads();
    if (wid != 0) return;
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = s_red[((0 * NT + j) * 4 + i) * 64 + lane];
        for (int w = 1; w < splits; ++w) s += s_red[((w * NT + j) * 4 + i) * 64 + lane];
        acc[j][i] = s;
      }
  }

  // ---- epilogue: lane holds rows row0 + 4*g4 + i, column (tile j) ... + m
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int orow = row0 + 4 * g4 + i;
    int pair = -1;
    if (grouped) {
      pair = g.row_to_pair[orow];
      if (pair < 0) continue;
    } else {
      if (orow >= g.M) continue;
      pair = orow;
    }
    if (g.epi == Epi::SITU) {
      const float inv_b = 1.0f / g.beta;
      const float inv_lb = g.lbeta > 0.0f ? 1.0f / g.lbeta : 0.0f;
#pragma unroll
      for (int j = 0; j < half; ++j) {
        const int col = nb * half * 16 + j * 16 + m;
        const float v = situ(acc[j][i], acc[j + half][i], g.beta, inv_b, g.lbeta, inv_lb);
        store_elt(g.out_elt, g.out, (size_t)orow * g.ldo + col, v);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int col = nb * NT * 16 + j * 16 + m;
        const float v = acc[j][i];
        if (g.epi == Epi::STORE) {
          store_elt(g.out_elt, g.out, (size_t)orow * g.ldo + col, v);
        } else if (g.epi == Epi::PAIR) {
          const float wgt = g.pair_w ? g.pair_w[pair] : 1.0f;
          reinterpret_cast<float*>(g.out)[(size_t)pair * g.ldo + col] = wgt * v;
        } else if (g.epi == Epi::TOKEN) {
          const float wgt = g.pair_w ? g.pair_w[pair] : 1.0f;
          store_elt(g.out_elt, g.out, (size_t)(pair / g.topk) * g.ldo + col, wgt * v);
        } else {   // ADD
          const size_t idx = (size_t)orow * g.ldo + col;
          const float add = g.add ? load_elt(g.out_elt, g.add, idx) : 0.0f;
          store_elt(g.out_elt, g.out, idx, add + v);
        }
      }
    }
  }
}

template <Elt ELT>
static hipError_t launch_elt(const StreamGemm& g, int n_out_cols, int live, hipStream_t stream) {
  using TR = EltTraits<ELT>;
  const int kchunks = g.Kd / TR::KCH;
  const int m_tiles = (g.M + 15) / 16;
  const bool situ = g.epi == Epi::SITU;
  const int tiles16 = n_out_cols / 16;   // output-column tiles (gate tiles for SituGLU)
  if (live < 1) live = 1;
  // tile columns per wave: as many as keep >= ~2048 waves alive
  int nt_out = 4;   // output tiles per wave (for SituGLU: gate tiles, each paired with its up tile)
  if (situ) nt_out = 2;
  while (nt_out > 1 && (tiles16 % nt_out != 0 || (long)live * (tiles16 / nt_out) < 2048)) nt_out >>= 1;
  const int n_blocks = tiles16 / nt_out;
  int splits = (int)((2048 + (long)live * n_blocks - 1) / ((long)live * n_blocks));
  splits = splits < 1 ? 1 : (splits > 8 ? 8 : splits);
  if (splits > kchunks) splits = kchunks;
  const dim3 grid((unsigned)(m_tiles * n_blocks)), block(64 * splits);
  const int NT = situ ? 2 * nt_out : nt_out;
  const size_t lds = splits > 1 ? (size_t)splits * NT * 4 * 64 * sizeof(float) : 0;
  switch (NT) {
    case 1: hipLaunchKernelGGL((stream_gemm_kernel<ELT, 1>), grid, block, lds, stream, g, n_blocks, kchunks); break;
    case 2: hipLaunchKernelGGL((stream_gemm_kernel<ELT, 2>), grid, block, lds, stream, g, n_blocks, kchunks); break;
    case 4: hipLaunchKernelGGL((stream_gemm_kernel<ELT, 4>), grid, block, lds, stream, g, n_blocks, kchunks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stream_gemm(const StreamGemm& g, Elt elt, int n_out_cols, int live_tiles, hipStream_t stream) {
  return elt == Elt::BF16 ? launch_elt<Elt::BF16>(g, n_out_cols, live_tiles, stream)
                          : launch_elt<Elt::F32>(g, n_out_cols, live_tiles, stream);
}

}  // namespace lmoe
