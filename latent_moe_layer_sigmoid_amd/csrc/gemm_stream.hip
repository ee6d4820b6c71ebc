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
// (and up to D - 1 further chunks) are issued before the current chunk's MFMAs. Up to 8 wavefronts of a workgroup split the K range; their fp32
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
// for lane l. Every load instruction reads 1 KB contiguous. POL is the cache policy: when
// each weight byte is read once in the launch the loads carry the non-temporal hint (the
// decode layer step measured about 5% faster with it); when several row tiles re-read the
// same weights they keep the default, so that the re-reads can hit the caches.
template <int POL>
LMOE_DEV Chunk load_chunk_w(rsrc_t r, uint32_t voff, uint32_t soff) {
  Chunk c;
  c.v[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POL));
  c.v[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 1024, soff, POL));
  c.v[2] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 2048, soff, POL));
  c.v[3] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 3072, soff, POL));
  return c;
}
constexpr int kPolDefault = 0;
constexpr int kPolStream = 2;   // nt

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

// MB (several blocks per wave): one segment, no split-K, no second phase. The wave walks
// nbw consecutive column blocks of its row tile; its ring runs on across block boundaries
// (the next block's first chunks are requested while the current block finishes), and
// each block's epilogue runs as soon as its last chunk has been consumed.
template <Elt ELT, int NT, bool DUAL, int D, bool MB, int POL>
__global__ __launch_bounds__(512) void stream_gemm_kernel(const StreamGemm g, int groups_total, int nbw, int nch0,
                                                          int nch1) {
  static_assert(!(MB && DUAL), "several blocks per wave: single phase only");
  using TR = EltTraits<ELT>;
  constexpr int CB = TR::KCH * TR::BYTES;   // bytes per chunk row (256)
  constexpr int NACC = DUAL ? 2 * NT : NT;
  extern __shared__ float s_red[];         // [splits][NACC][4][64] when splits > 1
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int splits = blockDim.x >> 6;
  const int mt = blockIdx.x / groups_total;
  const int nb_all = (blockIdx.x - mt * groups_total) * nbw;   // first column block of this workgroup
  const int row0 = mt * 16;
  if (row0 >= g.M) return;

  // ---- output segment of this workgroup (uniform)
  int s = 0;
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (i < g.nseg && nb_all >= g.seg[i].block0) s = i;
  const Seg sg = g.seg[s];
  const int nb = nb_all - sg.block0;
  const int nblk = MB ? min(nbw, sg.blocks - nb) : 1;
  const bool situ = sg.epi == Epi::SITU;

  const bool grouped = g.row_to_pair != nullptr;
  int e = 0;
  if (grouped) {
    e = g.tile_expert[row0 / g.tile_m];
    if (e < 0) return;
  }
  const int m = lane & 15;
  const int g4 = lane >> 4;

  // Start-up is a chain of dependent lookups (tile -> expert, row -> pair -> token row);
  // the row -> pair entries of the A row and of the four epilogue rows are requested
  // together, and the first weight chunk is requested as soon as the expert is known.
  int pair_a = 0, pair_o[4] = {0, 0, 0, 0};
  if (grouped) {
    pair_a = g.row_to_pair[row0 + m];
#pragma unroll
    for (int i = 0; i < 4; ++i) pair_o[i] = g.row_to_pair[row0 + 4 * g4 + i];
  }

  // ---- weight tiles: start of tile j's row group in the packed layout, plus the lane's 16 bytes.
  // The next column block's tiles start bstride bytes further (half or NT row groups on).
  const int half = NT / 2;
  const uint32_t w_bytes = (uint32_t)sg.n_total * (uint32_t)(g.Kd * TR::BYTES);   // one expert
  const rsrc_t w_rs = make_rsrc(reinterpret_cast<const char*>(sg.w) + (size_t)e * w_bytes, w_bytes);
  const uint32_t bstride = (uint32_t)(situ ? half : NT) * (uint32_t)nch0 * 4096u;
  uint32_t b_off[NT], b1_off[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int n0;
    if (situ)
      n0 = (j < half) ? nb * half * 16 + j * 16 : sg.n_out + nb * half * 16 + (j - half) * 16;
    else
      n0 = nb * NT * 16 + j * 16;
    b_off[j] = (uint32_t)(n0 / 16) * (uint32_t)nch0 * 4096u + lane * 16;
    b1_off[j] = (uint32_t)(n0 / 16) * (uint32_t)nch1 * 4096u + lane * 16;
  }
  rsrc_t w1_rs = w_rs;
  if (DUAL) {
    const uint32_t w1_bytes = (uint32_t)sg.n_total * (uint32_t)(g.Kd1 * TR::BYTES);
    w1_rs = make_rsrc(g.w1, w1_bytes);
  }

  // ---- K range of this wave (wave-uniform), over the chunks of both phases
  const int nch = nch0 + (DUAL ? nch1 : 0);
  const int wu = __builtin_amdgcn_readfirstlane(wid);
  const int v0 = (int)((long)nch * wu / splits);
  const int v1 = (int)((long)nch * (wu + 1) / splits);

  Chunk a[D], b[D][NT];   // ring of D chunks in flight
  if (v0 < v1) {   // first weight chunk (phase 0 unless the range starts in phase 1)
    if (!DUAL || v0 < nch0) {
#pragma unroll
      for (int j = 0; j < NT; ++j) b[0][j] = load_chunk_w<POL>(w_rs, b_off[j], (uint32_t)v0 * 4096u);
    } else {
#pragma unroll
      for (int j = 0; j < NT; ++j) b[0][j] = load_chunk_w<POL>(w1_rs, b1_off[j], (uint32_t)(v0 - nch0) * 4096u);
    }
  }

  // ---- A row of this lane
  int arow;
  if (grouped) {
    const uint64_t valid = __ballot(pair_a >= 0);
    if (valid == 0) return;                          // all-padding sub-tile (uniform per block)
    const int src = __ffsll((unsigned long long)valid) - 1;
    const int fill = __shfl(pair_a, src, WAVE);
    const int p = pair_a >= 0 ? pair_a : fill;
    const int r = pair_a >= 0 ? row0 + m : row0 + src;
    arow = g.a_by_row ? r : p / g.topk;
  } else {
    arow = min(row0 + m, g.M - 1);
  }
  const rsrc_t a_rs = make_rsrc(g.a, g.a_bytes);
  const uint32_t a_off = (uint32_t)arow * (uint32_t)(g.lda * TR::BYTES) + g4 * 16;
  rsrc_t a1_rs = a_rs;
  uint32_t a1_off = 0;
  if (DUAL) {
    a1_rs = make_rsrc(g.a1, g.a1_bytes);
    a1_off = (uint32_t)arow * (uint32_t)(g.lda1 * TR::BYTES) + g4 * 16;
  }

  // ---- epilogue operands, requested now so that their latency hides behind the K loop
  // (loaded in the epilogue, each would wait behind every load still in flight): the
  // combine weights of the lane's four rows (PAIR / TOKEN; four-tile waves, the grouped
  // FC2's shape) and the in-place addends (ADD; one-tile waves, the up projection's shape;
  // the lane reads the elements it writes). Other widths load them in the epilogue: the
  // registers held through the K loop would cost them a wave per SIMD.
  constexpr bool PW_PRE = NT == 4;
  float pw[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  if constexpr (PW_PRE) {
    if ((sg.epi == Epi::PAIR || sg.epi == Epi::TOKEN) && g.pair_w != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int orow = row0 + 4 * g4 + i;
        const int pair = grouped ? pair_o[i] : (orow < g.M ? orow : -1);
        if (pair >= 0) pw[i] = g.pair_w[pair];
      }
    }
  }
  constexpr bool ADD_PRE_OK = NT == 1 && !DUAL && !MB;
  const bool add_pre = ADD_PRE_OK && sg.epi == Epi::ADD && g.add != nullptr;
  float addv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (ADD_PRE_OK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int orow = row0 + 4 * g4 + i;
      const int col = nb * 16 + m;
      if (add_pre && orow < g.M && col < sg.n_out) addv[i] = load_elt(sg.out_elt, g.add, (size_t)orow * sg.ldo + col);
    }
  }

  floatx4 acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // ---- epilogue of column block nbk: lane holds rows row0 + 4*g4 + i, column (tile j) ... + m
  auto epilogue = [&](int nbk) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int orow = row0 + 4 * g4 + i;
      int pair = -1;
      if (grouped) {
        pair = pair_o[i];
        if (pair < 0) continue;
      } else {
        if (orow >= g.M) continue;
        pair = orow;
      }
      if (situ) {
        const float inv_b = 1.0f / g.beta;
        const float inv_lb = g.lbeta > 0.0f ? 1.0f / g.lbeta : 0.0f;
#pragma unroll
        for (int j = 0; j < half; ++j) {
          const int col = nbk * half * 16 + j * 16 + m;
          if (col >= sg.n_out) continue;   // partial last block of the segment
          const float v = situ_f(acc[j][i], acc[j + half][i], g.beta, inv_b, g.lbeta, inv_lb);
          store_elt(sg.out_elt, sg.out, (size_t)orow * sg.ldo + col, v);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int col = nbk * NT * 16 + j * 16 + m;
          if (col >= sg.n_out) continue;   // partial last block of the segment
          float v = acc[j][i];
          if (sg.epi == Epi::STORE) {
            store_elt(sg.out_elt, sg.out, (size_t)orow * sg.ldo + col, v);
          } else if (sg.epi == Epi::PAIR) {
            const float wgt = PW_PRE ? pw[i] : (g.pair_w ? g.pair_w[pair] : 1.0f);
            reinterpret_cast<float*>(sg.out)[(size_t)pair * sg.ldo + col] = wgt * v;
          } else if (sg.epi == Epi::TOKEN) {
            const float wgt = PW_PRE ? pw[i] : (g.pair_w ? g.pair_w[pair] : 1.0f);
            store_elt(sg.out_elt, sg.out, (size_t)(pair / g.topk) * sg.ldo + col, wgt * v);
          } else if (sg.epi == Epi::ADD) {
            const size_t idx = (size_t)orow * sg.ldo + col;
            const float add = add_pre ? addv[i] : (g.add ? load_elt(sg.out_elt, g.add, idx) : 0.0f);
            store_elt(sg.out_elt, sg.out, idx, add + v);
          } else if (DUAL) {   // ADD2: the first phase's result rounded to the output type, plus the second's
            if (sg.out_elt == Elt::BF16) v = bf16_to_f32(f32_to_bf16(v));
            store_elt(sg.out_elt, sg.out, (size_t)orow * sg.ldo + col, v + acc[NT + j][i]);
          }
        }
      }
    }
  };

  // Operands of chunk c (K chunk of the phase) of column block ib; the phase is wave-uniform,
  // so the selects below are scalar, and the block enters through the scalar offset.
  auto issue_at = [&](bool p1, uint32_t c, uint32_t ib, Chunk& ca, Chunk (&cb)[NT]) __attribute__((always_inline)) {
    ca = load_chunk_a(p1 ? a1_rs : a_rs, p1 ? a1_off : a_off, c * CB);
#pragma unroll
    for (int j = 0; j < NT; ++j)
      cb[j] = load_chunk_w<POL>(p1 ? w1_rs : w_rs, p1 ? b1_off[j] : b_off[j], c * 4096u + ib * bstride);
  };
  auto issue = [&](int v, Chunk& ca, Chunk (&cb)[NT]) __attribute__((always_inline)) {
    const bool p1 = DUAL && v >= nch0;
    issue_at(p1, (uint32_t)(p1 ? v - nch0 : v), 0u, ca, cb);
  };
  auto consume = [&](int v, const Chunk& ca, const Chunk (&cb)[NT]) __attribute__((always_inline)) {
    if (!DUAL || v < nch0) {
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = mfma_chunk<ELT>(ca, cb[j], acc[j]);
    } else {
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[NT + j] = mfma_chunk<ELT>(ca, cb[j], acc[NT + j]);
    }
  };

  // Ring of D chunk buffers: the chunk D - 1 places ahead is requested before the current
  // chunk is consumed. The request position stops at the wave's last chunk, so the final
  // requests re-read a chunk that is still cached instead of running past the range; they
  // are never consumed. sched_barrier keeps the compiler from sinking the requests below the
  // MFMAs that consume the older buffers (which would serialize every chunk on memory latency).
  if (MB) {
    // (ib, ic): next chunk to request; (cbk, cc): next chunk to consume. v0 = 0, v1 = nch0.
    a[0] = load_chunk_a(a_rs, a_off, 0u);
    int ib = 0, ic = 0;
    auto advance = [&]() __attribute__((always_inline)) {
      if (++ic == nch0) {
        if (ib + 1 < nblk) {
          ++ib;
          ic = 0;
        } else {
          ic = nch0 - 1;
        }
      }
    };
    advance();
    static_for<D - 2>([&](auto i) {
      constexpr int sl = decltype(i)::value + 1;
      issue_at(false, (uint32_t)ic, (uint32_t)ib, a[sl], b[sl]);
      advance();
    });
    int cbk = 0, cc = 0;
    bool more = true;
    while (more) {
      static_for<D>([&](auto i) {
        constexpr int sl = decltype(i)::value;
        if (!more) return;
        issue_at(false, (uint32_t)ic, (uint32_t)ib, a[(sl + D - 1) % D], b[(sl + D - 1) % D]);
        advance();
        __builtin_amdgcn_sched_barrier(0);
        consume(0, a[sl], b[sl]);
        __builtin_amdgcn_sched_barrier(0);
        if (++cc == nch0) {
          epilogue(nb + cbk);
#pragma unroll
          for (int j = 0; j < NACC; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
          cc = 0;
          if (++cbk >= nblk) more = false;
        }
      });
    }
    return;
  }

  if (v0 < v1) {
    if (!DUAL || v0 < nch0)
      a[0] = load_chunk_a(a_rs, a_off, (uint32_t)v0 * CB);
    else
      a[0] = load_chunk_a(a1_rs, a1_off, (uint32_t)(v0 - nch0) * CB);
    static_for<D - 2>([&](auto i) {
      constexpr int sl = decltype(i)::value + 1;
      issue(min(v0 + sl, v1 - 1), a[sl], b[sl]);
    });
    int v = v0;
    bool more = true;
    while (more) {
      static_for<D>([&](auto i) {
        constexpr int sl = decltype(i)::value;
        if (!more) return;
        issue(min(v + D - 1, v1 - 1), a[(sl + D - 1) % D], b[(sl + D - 1) % D]);
        __builtin_amdgcn_sched_barrier(0);
        consume(v, a[sl], b[sl]);
        __builtin_amdgcn_sched_barrier(0);
        if (++v >= v1) more = false;
      });
    }
  }

  // ---- split-K reduction in fixed wave order
  if (splits > 1) {
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_red[((wid * NACC + j) * 4 + i) * 64 + lane] = acc[j][i];
    __syncthreads();
    if (wid != 0) return;
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float t = s_red[(j * 4 + i) * 64 + lane];
        for (int w = 1; w < splits; ++w) t += s_red[((w * NACC + j) * 4 + i) * 64 + lane];
        acc[j][i] = t;
      }
  }
  epilogue(nb);
}

// Chunks in flight per wave (the ring depth).
template <int NT>
constexpr int depth_of() {
  return 2;
}

template <Elt ELT, int NT, int POL>
static void launch_pol(bool dual, int nbw, dim3 grid, dim3 block, size_t lds, hipStream_t stream, const StreamGemm& g,
                       int groups_total, int nch0, int nch1) {
  constexpr int D = depth_of<NT>();
  if (dual)
    hipLaunchKernelGGL((stream_gemm_kernel<ELT, NT, true, D, false, POL>), grid, block, lds, stream, g, groups_total,
                       1, nch0, nch1);
  else if (nbw > 1)
    hipLaunchKernelGGL((stream_gemm_kernel<ELT, NT, false, D, true, POL>), grid, block, lds, stream, g, groups_total,
                       nbw, nch0, nch1);
  else
    hipLaunchKernelGGL((stream_gemm_kernel<ELT, NT, false, D, false, POL>), grid, block, lds, stream, g, groups_total,
                       1, nch0, nch1);
}

template <Elt ELT, int NT>
static void launch_nt(bool dual, int nbw, dim3 grid, dim3 block, size_t lds, hipStream_t stream, const StreamGemm& g,
                      int groups_total, int nch0, int nch1) {
  if (g.weights_once)
    launch_pol<ELT, NT, kPolStream>(dual, nbw, grid, block, lds, stream, g, groups_total, nch0, nch1);
  else
    launch_pol<ELT, NT, kPolDefault>(dual, nbw, grid, block, lds, stream, g, groups_total, nch0, nch1);
}

// Waves a launch aims for (8 per CU). More, thinner waves measured slower: each wave
// pays a fixed start-up chain of dependent lookups before its loads stream.
constexpr long kTargetWaves = 2048;

template <Elt ELT>
static hipError_t launch_elt(StreamGemm g, int live, hipStream_t stream, long target_waves) {
  // Decode-sized grouped FC2 (per-pair products, every weight row met by one row tile):
  // K = d is short, so half as many waves, each walking twice as many column blocks, pay
  // the start-up of a wave over more bytes (T = 8, d = 512, L = 2048: FC2 + combine 59.4 ->
  // 57.8 us; 3072 or 4096 waves slower).
  const bool short_k_pairs = g.row_to_pair && g.weights_once && g.nseg == 1 && g.seg[0].epi == Epi::PAIR;
  const long tw = target_waves > 0 ? target_waves : (short_k_pairs ? kTargetWaves / 2 : kTargetWaves);
  using TR = EltTraits<ELT>;
  if (!g.row_to_pair) g.weights_once = g.M <= 16;   // dense: one row tile reads every weight
  const bool dual = g.nseg == 1 && g.seg[0].epi == Epi::ADD2;
  const int nch0 = g.Kd / TR::KCH;
  const int nch1 = dual ? g.Kd1 / TR::KCH : 0;
  const int m_tiles = (g.M + 15) / 16;
  if (live < 1) live = 1;
  // Columns per wave: NT tiles of 16 (a SituGLU segment pairs NT/2 gate tiles with their
  // up tiles; a segment's last block may be partial). Take the largest NT that still gives
  // tw live waves (kTargetWaves unless the caller asks for another count), else the
  // smallest allowed; then split K over up to 8 waves of a workgroup to reach that count.
  // With more live waves than the target (one segment, one phase), a wave takes several
  // consecutive column blocks instead.
  bool any_situ = false;
  for (int i = 0; i < g.nseg; ++i) any_situ |= g.seg[i].epi == Epi::SITU;
  auto blocks_of = [&](int i, int NT) {
    const int tiles = g.seg[i].n_out / 16;
    const int per = g.seg[i].epi == Epi::SITU ? NT / 2 : NT;
    return (tiles + per - 1) / per;
  };
  int NT = 0, blocks_total = 0;
  for (int cand : {4, 2, 1}) {
    if (any_situ && cand < 2) break;
    int t = 0;
    for (int i = 0; i < g.nseg; ++i) t += blocks_of(i, cand);
    NT = cand;
    blocks_total = t;
    if ((long)live * t >= tw) break;
  }
  for (int i = 0, b0 = 0; i < g.nseg; ++i) {
    g.seg[i].blocks = blocks_of(i, NT);
    g.seg[i].block0 = b0;
    b0 += g.seg[i].blocks;
  }
  int splits = (int)((tw + (long)live * blocks_total - 1) / ((long)live * blocks_total));
  splits = splits < 1 ? 1 : (splits > 8 ? 8 : splits);
  if (splits > nch0 + nch1) splits = nch0 + nch1;
  int nbw = 1;
  if (splits == 1 && !dual && g.nseg == 1) {
    nbw = (int)((long)live * blocks_total / tw);
    nbw = nbw < 1 ? 1 : (nbw > blocks_total ? blocks_total : nbw);
  }
  const int groups_total = (blocks_total + nbw - 1) / nbw;
  const dim3 grid((unsigned)(m_tiles * groups_total)), block(64 * splits);
  const size_t lds = splits > 1 ? (size_t)splits * (dual ? 2 : 1) * NT * 4 * 64 * sizeof(float) : 0;
  switch (NT) {
    case 1: launch_nt<ELT, 1>(dual, nbw, grid, block, lds, stream, g, groups_total, nch0, nch1); break;
    case 2: launch_nt<ELT, 2>(dual, nbw, grid, block, lds, stream, g, groups_total, nch0, nch1); break;
    default: launch_nt<ELT, 4>(dual, nbw, grid, block, lds, stream, g, groups_total, nch0, nch1); break;
  }
  return hipGetLastError();
}

hipError_t launch_stream_gemm(StreamGemm g, Elt elt, int live_tiles, hipStream_t stream, long target_waves) {
  return elt == Elt::BF16 ? launch_elt<Elt::BF16>(g, live_tiles, stream, target_waves)
                          : launch_elt<Elt::F32>(g, live_tiles, stream, target_waves);
}

}  // namespace lmoe
