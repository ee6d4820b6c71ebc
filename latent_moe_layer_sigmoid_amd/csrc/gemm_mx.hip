// MX expert GEMMs for gfx950: MXFP8 (E4M3) activations x MXFP4 (E2M1) weights on the
// scaled matrix core (v_mfma_scale_f32_16x16x128_f8f6f4), fp32 accumulation of the
// dequantized products (vLLM PR 50088, commit 5: the gated activation acts on the
// dequantized gate/up; TensorRT-LLM PR 20541, "Description": the MXE4M3 x MXE2M1 expert
// runner; commit 3 of the vLLM PR: apply the activation, then requantize to FP8).
//
// Operand layout of one 16x16x128 scaled MFMA (measured on gfx950 with one-hot probes):
// lane l = 16g + r holds row / column r; an e2m1 B lane holds K [32g, 32g + 32) of the
// 128 in nibble order; an e4m3 A lane holds K [16g, 16g + 16) in bytes 0..15 and
// [64 + 16g, 64 + 16g + 16) in bytes 16..31; the e8m0 scale a lane supplies (for A and for
// B) covers K block [32g, 32g + 32). Loading A that way makes the hardware K order the
// natural one, so the MX blocks of the data line up with the scales.
//
// Grouped expert tiles of 16 rows (or 32 when the permutation's tile is a multiple of 32:
// two row groups then share every weight fragment, halving weight traffic per row), one
// wavefront per (tile, column block) in FC1 and per (tile, two neighbouring column blocks)
// in FC2, NT tiles of 16 columns per block. A pipeline step is
// 256 K elements = two scaled MFMAs per row group: per lane 2 x 32 fp8 bytes of each
// activation row (row-major) and, per weight tile, 2 x 16 bytes of packed e2m1 codes (one
// contiguous 1 KB per wave-wide load; layout written by lmoe_pack_mxfp4_weights) plus one
// dword holding the lane's four weight scales of the 512-wide stage.
// Epilogues: SituGLU on the fp32 accumulators followed by MXFP8 requantization of each
// 32 consecutive outputs (2 gate tiles x 16 lanes share one block: amax by butterfly
// over the 16 lanes), or the weighted per-pair store of FC2.
#include "common.h"
#include "kernels.h"

namespace lmoe {

// column blocks an FC2 wavefront walks (measured at T = 1024, d = 512, L = 2048: FC2 +
// combine 183 / 167 / 169 / 179 us for 1 / 2 / 4 / 8)
constexpr int MX_FC2_BLOCKS_PER_WAVE = 2;
// consecutive FC1 row tiles placed on one XCD, so that an expert's two 32-row tiles read its
// weights into one L2 (measured at T = 1024: FC1 reads 1.14 / 1.04 / 0.97 GB and takes
// 255 / 253 / 254 us for 1 / 2 / 4)
constexpr int MX_FC1_TILES_PER_XCD = 2;

template <int NT, int R>
struct MxStep {
  uint4 a[R][4];     // A codes of row group r: MFMA u uses a[r][2u] (K 16g..) and a[r][2u+1] (K 64+16g..)
  uint32_t sa[R][2]; // A scales (byte in bits 0..7)
  uint4 b[NT][2];    // B codes: MFMA u uses b[j][u] (16 bytes = 32 e2m1)
  uint32_t sb[NT];   // B scales of the stage: byte q = 2h + u
};

// WALK (FC2 only): each wavefront walks blocks_per_wave column blocks, storing a block's
// products while the next block's first step loads; a kernel of its own, so that the
// registers of the SituGLU epilogue do not count against it.
template <int NT, int R, bool WALK>
__device__ __forceinline__ void mx_gemm_body(const StreamGemm& g, int blocks_total, int nsteps, int grouped_waves,
                                             int blocks_per_wave) {
  const int lane = threadIdx.x & 63;
  int mt, nb;
  if (grouped_waves) {
    // A workgroup's 4 wavefronts take 4 neighbouring column blocks of one row tile, so they
    // request the same activation rows on one CU; the workgroups of a row tile run on one
    // XCD (workgroup b runs on XCD b % 8), runs of MX_FC1_TILES_PER_XCD consecutive row tiles
    // on the XCDs in turn, so that each tile's activation rows and most experts' weights
    // cross into one L2 only and the tiles holding rows (the first ones) spread over all
    // XCDs.
    const int nwb = (blocks_total + 3) / 4;
    const int j = (int)(blockIdx.x >> 3);
    const int jt = j / nwb;                 // this XCD's jt-th row tile
    mt = ((jt / MX_FC1_TILES_PER_XCD) * 8 + (int)(blockIdx.x & 7)) * MX_FC1_TILES_PER_XCD + jt % MX_FC1_TILES_PER_XCD;
    nb = (j - jt * nwb) * 4 + (int)(threadIdx.x >> 6);
    if (nb >= blocks_total) return;
  } else {
    // one wavefront per workgroup, walking blocks_per_wave consecutive column blocks of a
    // row tile (FC2 only: the SituGLU epilogue takes one block per wavefront)
    const int wpt = (blocks_total + blocks_per_wave - 1) / blocks_per_wave;
    mt = blockIdx.x / wpt;
    nb = (blockIdx.x - mt * wpt) * blocks_per_wave;
  }
  const int nblk_w = WALK ? min(blocks_per_wave, blocks_total - nb) : 1;   // column blocks walked
  const int row0 = mt * 16 * R;   // R row groups of 16 share every weight fragment
  if (row0 >= g.M) return;
  const Seg sg = g.seg[0];
  const bool situ = sg.epi == Epi::SITU_MX;
  const int e = g.tile_expert[row0 / g.tile_m];
  if (e < 0) return;
  const int m = lane & 15;
  const int g4 = lane >> 4;
  const int Kd = g.Kd;
  const int nst = Kd / 512;

  int pair_o[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) pair_o[r][i] = g.row_to_pair[row0 + 16 * r + 4 * g4 + i];
  // combine weights of the lane's output rows (FC2), requested now so that their latency
  // hides behind the K loop
  float pw[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pw[r][i] = (!situ && g.pair_w != nullptr && pair_o[r][i] >= 0) ? g.pair_w[pair_o[r][i]] : 1.0f;

  // weight tiles (packed codes and scales of expert e)
  const int half = NT / 2;
  const uint32_t wc_bytes = (uint32_t)sg.n_total * (uint32_t)(Kd / 2);
  const uint32_t ws_bytes = (uint32_t)sg.n_total * (uint32_t)(Kd / 32);
  const rsrc_t wc_rs = make_rsrc(reinterpret_cast<const uint8_t*>(sg.w) + (size_t)e * wc_bytes, wc_bytes);
  const rsrc_t ws_rs = make_rsrc(g.w_scale + (size_t)e * ws_bytes, ws_bytes);
  uint32_t n16[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n0 = situ ? ((j < half) ? nb * half * 16 + j * 16 : sg.n_out + nb * half * 16 + (j - half) * 16)
                        : nb * NT * 16 + j * 16;
    n16[j] = (uint32_t)(n0 / 16);
  }

  // activation rows: a pad row reads the tile's first row; a tile whose first row is a pad
  // holds only pads (pads close each expert's segment)
  const int first = g.row_to_pair[row0];
  if (first < 0) return;
  const rsrc_t ac_rs = make_rsrc(g.a, g.a_bytes);
  const rsrc_t as_rs = make_rsrc(g.a_scale, g.a_scale_bytes);
  uint32_t ac_off[R], as_off[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int pa = g.row_to_pair[row0 + 16 * r + m];
    const bool real = pa >= 0;
    const int arow = g.a_by_row ? (real ? row0 + 16 * r + m : row0) : (real ? pa : first) / g.topk;
    ac_off[r] = (uint32_t)arow * (uint32_t)Kd + g4 * 16;
    as_off[r] = (uint32_t)arow * (uint32_t)(Kd / 32) + g4;
  }

  // step t of the walk: K stage s of column block t / nsteps (nsteps is even: K is a
  // multiple of 512)
  auto issue = [&](int t, MxStep<NT, R>& st) {
    const int bi = t / nsteps;
    const int tl = t - bi * nsteps;
    const int s = tl >> 1, h = tl & 1;
    const uint32_t nbase = (uint32_t)(bi * NT);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = 2 * h + u;
      const uint32_t ko = (uint32_t)(s * 512 + q * 128);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        st.a[r][2 * u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ac_rs, ac_off[r], ko, 0));
        st.a[r][2 * u + 1] =
            __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ac_rs, ac_off[r] + 64, ko, 0));
        st.sa[r][u] = __builtin_amdgcn_raw_buffer_load_b8(as_rs, as_off[r], (uint32_t)(s * 16 + q * 4), 0);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j)
        st.b[j][u] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(wc_rs, lane * 16, ((n16[j] + nbase) * nst + s) * 4096u + q * 1024u, 0));
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
      st.sb[j] = __builtin_amdgcn_raw_buffer_load_b32(ws_rs, lane * 4, ((n16[j] + nbase) * nst + s) * 256u, 0);
  };

  floatx4 acc[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[r][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto consume = [&](int t, const MxStep<NT, R>& st) {
    const int h = t & 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const intx8 av = {(int)st.a[r][2 * u].x,     (int)st.a[r][2 * u].y,     (int)st.a[r][2 * u].z,
                          (int)st.a[r][2 * u].w,     (int)st.a[r][2 * u + 1].x, (int)st.a[r][2 * u + 1].y,
                          (int)st.a[r][2 * u + 1].z, (int)st.a[r][2 * u + 1].w};
        const int sa = (int)(st.sa[r][u] & 0xFFu);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const intx8 bv = {(int)st.b[j][u].x, (int)st.b[j][u].y, (int)st.b[j][u].z, (int)st.b[j][u].w, 0, 0, 0, 0};
          const int sb = (int)((st.sb[j] >> (8 * (2 * h + u))) & 0xFFu);
          acc[r][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[r][j], 0, 4, 0, sa, 0, sb);
        }
      }
    }
  };

  // ---- epilogue of column block nbc: row group r, lane holds rows row0 + 16 r + 4*g4 + i,
  // column (tile j) ... + m
  auto epilogue = [&](int nbc) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!WALK && situ) {
        const float inv_b = 1.0f / g.beta;
        const float inv_lb = g.lbeta > 0.0f ? 1.0f / g.lbeta : 0.0f;
        const int nblk = sg.n_out / 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int orow = row0 + 16 * r + 4 * g4 + i;
          float v[half];
          float amax = 0.0f;
#pragma unroll
          for (int j = 0; j < half; ++j) {
            v[j] = situ_f(acc[r][j][i], acc[r][j + half][i], g.beta, inv_b, g.lbeta, inv_lb);
            amax = fmaxf(amax, fabsf(v[j]));
          }
          // one MX block = the 32 columns of this wave (NT/2 == 2 gate tiles x 16 lanes)
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, WAVE));
          const int X = mx_e4m3_exponent(amax);
          if (pair_o[r][i] < 0) continue;
          uint8_t* act = reinterpret_cast<uint8_t*>(sg.out) + (size_t)orow * sg.ldo;
#pragma unroll
          for (int j = 0; j < half; ++j)
            act[nbc * half * 16 + j * 16 + m] = (uint8_t)e4m3_encode(__builtin_ldexpf(v[j], -X));
          if (m == 0) g.out_scale[(size_t)orow * nblk + nbc] = (uint8_t)(X + 127);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pair = pair_o[r][i];
          if (pair < 0) continue;
          const float wgt = pw[r][i];
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const int col = nbc * NT * 16 + j * 16 + m;
            if (sg.epi == Epi::PAIR)
              reinterpret_cast<float*>(sg.out)[(size_t)pair * sg.ldo + col] = wgt * acc[r][j][i];
            else if (sg.out_elt == Elt::F32)   // TOKEN (K == 1)
              reinterpret_cast<float*>(sg.out)[(size_t)(pair / g.topk) * sg.ldo + col] = wgt * acc[r][j][i];
            else
              reinterpret_cast<uint16_t*>(sg.out)[(size_t)(pair / g.topk) * sg.ldo + col] = f32_to_bf16(wgt * acc[r][j][i]);
          }
        }
      }
    }
  };

  if constexpr (!WALK) {
    MxStep<NT, R> s0, s1;
    issue(0, s0);
    int t = 0;
    while (true) {
      issue(min(t + 1, nsteps - 1), s1);
      __builtin_amdgcn_sched_barrier(0);
      consume(t, s0);
      __builtin_amdgcn_sched_barrier(0);
      if (++t >= nsteps) break;
      issue(min(t + 1, nsteps - 1), s0);
      __builtin_amdgcn_sched_barrier(0);
      consume(t, s1);
      __builtin_amdgcn_sched_barrier(0);
      if (++t >= nsteps) break;
    }
    epilogue(nb);
  } else {
    // two steps per trip (nsteps is even), so that a column block ends after the second;
    // the next block's first step is already in flight during its epilogue
    const int total = nblk_w * nsteps;
    MxStep<NT, R> s0, s1;
    issue(0, s0);
    int t = 0, bi = 0;
    while (true) {
      issue(min(t + 1, total - 1), s1);
      __builtin_amdgcn_sched_barrier(0);
      consume(t, s0);
      __builtin_amdgcn_sched_barrier(0);
      ++t;
      issue(min(t + 1, total - 1), s0);
      __builtin_amdgcn_sched_barrier(0);
      consume(t, s1);
      __builtin_amdgcn_sched_barrier(0);
      ++t;
      if (t == (bi + 1) * nsteps) {
        epilogue(nb + bi);
        if (t >= total) break;
        ++bi;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int j = 0; j < NT; ++j) acc[r][j] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
}

template <int NT, int R>
__global__ __launch_bounds__(256) void stream_gemm_mx_kernel(const StreamGemm g, int blocks_total, int nsteps,
                                                             int grouped_waves) {
  mx_gemm_body<NT, R, false>(g, blocks_total, nsteps, grouped_waves, 1);
}

// two wavefronts per SIMD asked for explicitly: left to itself the compiler gives the walk
// more registers than that allows
template <int NT, int R>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void stream_gemm_mx_walk_kernel(
    const StreamGemm g, int blocks_total, int nsteps, int blocks_per_wave) {
  mx_gemm_body<NT, R, true>(g, blocks_total, nsteps, 0, blocks_per_wave);
}

hipError_t launch_stream_gemm_mx(StreamGemm g, int live, hipStream_t stream) {
  (void)live;
  const int nsteps = g.Kd / 256;
  // 32 rows per wavefront when expert tiles are a multiple of 32 rows (each weight fragment
  // then feeds two scaled MFMAs), else 16
  const int R = g.tile_m % 32 == 0 ? 2 : 1;
  const int m_tiles = (g.M + 16 * R - 1) / (16 * R);
  // SituGLU + requant needs 32 gate columns per wave (one MX block): 2 gate + 2 up tiles.
  constexpr int NT = 4;
  const int tiles = g.seg[0].n_out / 16;
  const int blocks = g.seg[0].epi == Epi::SITU_MX ? tiles / (NT / 2) : tiles / NT;
  g.seg[0].blocks = blocks;
  g.seg[0].block0 = 0;
  g.nseg = 1;
  // FC1 (long K: 64 KB of activation rows per 32-row tile): workgroups of 4 wavefronts
  // (4 column blocks of one row tile), whole rounds of 8 row tiles (one per XCD), the ids
  // past the tiles returning at once. FC2 (K = d: 16 KB per tile) measured faster with one
  // wavefront per workgroup.
  const bool grouped_waves = g.seg[0].epi == Epi::SITU_MX;
  // FC2 wavefronts walk MX_FC2_BLOCKS_PER_WAVE column blocks each, loading the next block
  // while they store the last one's products (fewer, longer-lived waves: each one's first
  // load latency is paid once per walk)
  const int bpw = grouped_waves ? 1 : MX_FC2_BLOCKS_PER_WAVE;
  const unsigned grid = grouped_waves ? (unsigned)(((m_tiles + 8 * MX_FC1_TILES_PER_XCD - 1) / (8 * MX_FC1_TILES_PER_XCD)) *
                                                   8 * MX_FC1_TILES_PER_XCD * ((blocks + 3) / 4))
                                      : (unsigned)(m_tiles * ((blocks + bpw - 1) / bpw));
  const unsigned threads = grouped_waves ? 256 : 64;
  if (grouped_waves) {
    if (R == 2)
      hipLaunchKernelGGL((stream_gemm_mx_kernel<NT, 2>), dim3(grid), dim3(threads), 0, stream, g, blocks, nsteps, 1);
    else
      hipLaunchKernelGGL((stream_gemm_mx_kernel<NT, 1>), dim3(grid), dim3(threads), 0, stream, g, blocks, nsteps, 1);
  } else {
    if (R == 2)
      hipLaunchKernelGGL((stream_gemm_mx_walk_kernel<NT, 2>), dim3(grid), dim3(threads), 0, stream, g, blocks, nsteps,
                         bpw);
    else
      hipLaunchKernelGGL((stream_gemm_mx_walk_kernel<NT, 1>), dim3(grid), dim3(threads), 0, stream, g, blocks, nsteps,
                         bpw);
  }
  return hipGetLastError();
}

}  // namespace lmoe
