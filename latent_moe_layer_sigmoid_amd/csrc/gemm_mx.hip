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

// ---- FC1 with the activation rows staged in LDS (32-row tiles) -----------------------
// A workgroup's 4 wavefronts compute 4 neighbouring column blocks of one 32-row tile and
// need the same activation rows. Per 256-wide K step the workgroup copies those rows
// (32 x 256 e4m3 bytes) and their e8m0 scales (32 x 8 bytes) into an LDS slot once, by
// buffer-to-LDS copies, and every wavefront reads its fragments from there; only the
// weights go straight to registers. This halves the bytes a wavefront requests (the data
// path from the L1 into registers, busy 86% of the time with every wavefront loading its
// own copy of the rows, is what held the kernel). The rows sit in LDS 256 bytes apart,
// with the 16-byte chunk c of row j stored at position c ^ (j % 16), so that the 16 lanes
// reading one chunk of 16 consecutive rows hit 16 different bank groups.
constexpr int MXL_NS = 4;                         // LDS slots (steps)
constexpr int MXL_D = 3;                          // steps in flight ahead of the one computed
constexpr int MXL_SLOT = 32 * 256 + 32 * 8;       // one step: 32 rows x 256 codes + 32 x 8 scales
constexpr int MXL_DMA = 3;                        // buffer-to-LDS copies per wavefront per step
typedef unsigned mx_u32x4 __attribute__((ext_vector_type(4)));

template <int NT>
struct MxB {       // the weight operands of one step
  uint4 b[NT][2];
  uint32_t sb[NT];
};

template <int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void mx_fc1_lds_kernel(
    const StreamGemm g, int blocks_total, int nsteps) {
  __shared__ __attribute__((aligned(1024))) char smem[MXL_NS * MXL_SLOT];
  constexpr int R = 2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // tile and column block: the same placement as the register-only kernel (a row tile's
  // workgroups on one XCD, runs of MX_FC1_TILES_PER_XCD consecutive tiles per XCD)
  const int nwb = (blocks_total + 3) / 4;
  const int jb = (int)(blockIdx.x >> 3);
  const int jt = jb / nwb;
  const int mt = ((jt / MX_FC1_TILES_PER_XCD) * 8 + (int)(blockIdx.x & 7)) * MX_FC1_TILES_PER_XCD + jt % MX_FC1_TILES_PER_XCD;
  const int nb = (jb - jt * nwb) * 4 + wave;
  const bool active = nb < blocks_total;   // every wavefront copies and meets the barriers
  const int row0 = mt * 32;
  if (row0 >= g.M) return;
  const int e = __builtin_amdgcn_readfirstlane(g.tile_expert[row0 / g.tile_m]);
  if (e < 0) return;
  const int first = __builtin_amdgcn_readfirstlane(g.row_to_pair[row0]);
  if (first < 0) return;                  // a tile whose first row is a pad holds only pads
  const Seg sg = g.seg[0];
  const int m = lane & 15, g4 = lane >> 4;
  const int Kd = g.Kd;
  const int nst = Kd / 512;
  const int half = NT / 2;

  int pair_o[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) pair_o[r][i] = g.row_to_pair[row0 + 16 * r + 4 * g4 + i];

  // weights of expert e (codes and scales, packed)
  const uint32_t wc_bytes = __builtin_amdgcn_readfirstlane((uint32_t)sg.n_total * (uint32_t)(Kd / 2));
  const uint32_t ws_bytes = __builtin_amdgcn_readfirstlane((uint32_t)sg.n_total * (uint32_t)(Kd / 32));
  const rsrc_t wc_rs = make_rsrc(uniform_ptr(reinterpret_cast<const uint8_t*>(sg.w) + (size_t)e * wc_bytes), wc_bytes);
  const rsrc_t ws_rs = make_rsrc(uniform_ptr(g.w_scale + (size_t)e * ws_bytes), ws_bytes);
  uint32_t n16[NT];
  const int nbw = active ? nb : 0;        // inactive wavefronts load block 0 (never used)
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n0 = (j < half) ? nbw * half * 16 + j * 16 : sg.n_out + nbw * half * 16 + (j - half) * 16;
    n16[j] = (uint32_t)(n0 / 16);
  }

  // ---- copies of step t: rows 8 wave + 4 i + lane / 16 (i = 0, 1), 16 bytes each: the
  // lane fills position lane % 16 of its row with chunk (lane % 16) ^ (row % 16); scales:
  // every wavefront copies all 32 rows' 8 bytes (lane: row lane / 2, 4 bytes), the same
  // bytes to the same place, so that all wavefronts issue the same loads per step
  const rsrc_t ac_rs = make_rsrc(uniform_ptr(g.a), __builtin_amdgcn_readfirstlane(g.a_bytes));
  const rsrc_t as_rs = make_rsrc(uniform_ptr(g.a_scale), __builtin_amdgcn_readfirstlane(g.a_scale_bytes));
  auto a_row = [&](int p) { return (p >= 0 ? p : first) / g.topk; };   // a pad reads the tile's first row
  int cp_row[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) cp_row[i] = g.row_to_pair[row0 + 8 * wave + 4 * i + (lane >> 4)];
  const int sc_row = g.row_to_pair[row0 + (lane >> 1)];
  uint32_t dma_off[2], sdma_off;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = 8 * wave + 4 * i + (lane >> 4);
    dma_off[i] = (uint32_t)a_row(cp_row[i]) * (uint32_t)Kd + (uint32_t)(((lane & 15) ^ (j & 15)) * 16);
  }
  sdma_off = (uint32_t)a_row(sc_row) * (uint32_t)(Kd / 32) + (uint32_t)(lane & 1) * 4u;
  auto copy_step = [&](int t) __attribute__((always_inline)) {
    const int tc = min(t, nsteps - 1);   // past the end: a copy of the last step (never read)
    char* slot = smem + (t % MXL_NS) * MXL_SLOT;
    to_lds(ac_rs, slot + (8 * wave + 0) * 256, dma_off[0], (uint32_t)tc * 256u);
    to_lds(ac_rs, slot + (8 * wave + 4) * 256, dma_off[1], (uint32_t)tc * 256u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(as_rs, (lds_void*)(slot + 32 * 256), 4, sdma_off, (uint32_t)tc * 8u, 0,
                                             0);   // 64 lanes x 4 bytes at slot + 32 * 256 + 4 lane
  };
  // weights of step t: 2 x 16 bytes per tile + the lane's scale dword of the 512-wide stage
  auto load_b = [&](int t, MxB<NT>& st) __attribute__((always_inline)) {
    const int tc = min(t, nsteps - 1);
    const int s = tc >> 1, h = tc & 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = 2 * h + u;
#pragma unroll
      for (int j = 0; j < NT; ++j)
        st.b[j][u] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(wc_rs, lane * 16, (n16[j] * nst + s) * 4096u + q * 1024u, 0));
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
      st.sb[j] = __builtin_amdgcn_raw_buffer_load_b32(ws_rs, lane * 4, (n16[j] * nst + s) * 256u, 0);
  };
  // ---- fragment reads of a step: row 16 r + m, chunks 8 u + 4 v + g4 (v = 0, 1) and the
  // scale byte u * 4 + g4 of the row's 8. The twelve addresses (slot 0) stay in registers
  // for the whole loop; the slot is an immediate offset (the loop is unrolled by the ring).
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  uint32_t ra[R][2][2], rs[R][2];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int v = 0; v < 2; ++v)
        ra[r][u][v] = lds_base + (uint32_t)((16 * r + m) * 256 + (((8 * u + 4 * v + g4) ^ m) * 16));
      rs[r][u] = lds_base + (uint32_t)(32 * 256 + (16 * r + m) * 8 + u * 4 + g4);
    }
  // all twelve reads of one step in one asm statement that also waits for them, so that no
  // result register is taken before its data has arrived
  auto read_a = [&ra, &rs](auto SLOT, mx_u32x4 (&a)[R][2][2], uint32_t (&sa)[R][2]) __attribute__((always_inline)) {
    constexpr int O = decltype(SLOT)::value * MXL_SLOT;
    asm volatile(
        "ds_read_b128 %0, %12 offset:%24\n"
        "ds_read_b128 %1, %13 offset:%24\n"
        "ds_read_b128 %2, %14 offset:%24\n"
        "ds_read_b128 %3, %15 offset:%24\n"
        "ds_read_b128 %4, %16 offset:%24\n"
        "ds_read_b128 %5, %17 offset:%24\n"
        "ds_read_b128 %6, %18 offset:%24\n"
        "ds_read_b128 %7, %19 offset:%24\n"
        "ds_read_u8 %8, %20 offset:%24\n"
        "ds_read_u8 %9, %21 offset:%24\n"
        "ds_read_u8 %10, %22 offset:%24\n"
        "ds_read_u8 %11, %23 offset:%24\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0][0][0]), "=&v"(a[0][0][1]), "=&v"(a[0][1][0]), "=&v"(a[0][1][1]), "=&v"(a[1][0][0]),
          "=&v"(a[1][0][1]), "=&v"(a[1][1][0]), "=&v"(a[1][1][1]), "=&v"(sa[0][0]), "=&v"(sa[0][1]),
          "=&v"(sa[1][0]), "=&v"(sa[1][1])
        : "v"(ra[0][0][0]), "v"(ra[0][0][1]), "v"(ra[0][1][0]), "v"(ra[0][1][1]), "v"(ra[1][0][0]),
          "v"(ra[1][0][1]), "v"(ra[1][1][0]), "v"(ra[1][1][1]), "v"(rs[0][0]), "v"(rs[0][1]), "v"(rs[1][0]),
          "v"(rs[1][1]), "i"(O)
        : "memory");
  };

  floatx4 acc[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[r][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](int t, const mx_u32x4 (&a)[R][2][2], const uint32_t (&sa)[R][2], const MxB<NT>& st)
      __attribute__((always_inline)) {
    const int h = t & 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const intx8 av = {(int)a[r][u][0][0], (int)a[r][u][0][1], (int)a[r][u][0][2], (int)a[r][u][0][3],
                          (int)a[r][u][1][0], (int)a[r][u][1][1], (int)a[r][u][1][2], (int)a[r][u][1][3]};
        const int sav = (int)(sa[r][u] & 0xFFu);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const intx8 bv = {(int)st.b[j][u].x, (int)st.b[j][u].y, (int)st.b[j][u].z, (int)st.b[j][u].w, 0, 0, 0, 0};
          const int sb = (int)((st.sb[j] >> (8 * (2 * h + u))) & 0xFFu);
          acc[r][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[r][j], 0, 4, 0, sav, 0, sb);
        }
      }
    }
  };

  // ---- pipeline. Issue order per wavefront: copies of steps 0 .. D-1, weights of step 0;
  // then per step t: copies of step t + D, weights of step t + 1 (both clamped to the last
  // step, so every step issues the same number of loads). At the top of step t this
  // wavefront's copies of step t are done once at most N(t) later loads are outstanding:
  // N(t) = 3 D + 9 + 12 t for t < D (issued in the prologue), 15 D - 3 after.
  static_assert(MXL_D == 3 && MXL_DMA == 3 && NT == 4, "the wait counts below assume these");
  auto wait_copies = [&](int t) __attribute__((always_inline)) {
    if (t == 0)
      __builtin_amdgcn_s_waitcnt(waitcnt(18, 15));
    else if (t == 1)
      __builtin_amdgcn_s_waitcnt(waitcnt(30, 15));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt(42, 15));
  };
#pragma unroll
  for (int t = 0; t < MXL_D; ++t) copy_step(t);
  __builtin_amdgcn_sched_barrier(0);
  MxB<NT> b0, b1;
  load_b(0, b0);
  __builtin_amdgcn_sched_barrier(0);
  auto step = [&](int t, auto SLOT, MxB<NT>& cur, MxB<NT>& nxt) __attribute__((always_inline)) {
    wait_copies(t);
    lds_barrier();     // every wavefront's copies of step t have landed; slot t - 1 is free
    mx_u32x4 a[R][2][2];
    uint32_t sa[R][2];
    read_a(SLOT, a, sa);
    __builtin_amdgcn_sched_barrier(0);
    copy_step(t + MXL_D);
    __builtin_amdgcn_sched_barrier(0);
    load_b(t + 1, nxt);
    __builtin_amdgcn_sched_barrier(0);
    consume(t, a, sa, cur);   // (an inactive wavefront computes block 0 and stores nothing)
  };
  // unrolled by the ring (slot = t % 4 is then a constant); nsteps is even. The common
  // K = 2048 (8 steps) is unrolled completely: with no loop back edge the registers of a
  // step's fragments are never renamed onto loads still in flight, which would otherwise
  // force a wait on them.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  if (nsteps == 8) {
    static_for<8>([&](auto T) __attribute__((always_inline)) {
      constexpr int tt = decltype(T)::value;
      if constexpr (tt % 2 == 0)
        step(tt, std::integral_constant<int, tt % MXL_NS>{}, b0, b1);
      else
        step(tt, std::integral_constant<int, tt % MXL_NS>{}, b1, b0);
    });
  } else {
    for (int t = 0; t < nsteps; t += 4) {
      step(t, S0{}, b0, b1);
      step(t + 1, S1{}, b1, b0);
      if (t + 2 >= nsteps) break;
      step(t + 2, S2{}, b0, b1);
      step(t + 3, S3{}, b1, b0);
    }
  }
  // the copies past the last step must land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
  if (!active) return;

  // ---- epilogue: SituGLU of the fp32 accumulators and MXFP8 requantization of each 32
  // outputs (this wavefront's 2 gate tiles x 16 lanes: amax by butterfly over 16 lanes)
  const float inv_b = 1.0f / g.beta;
  const float inv_lb = g.lbeta > 0.0f ? 1.0f / g.lbeta : 0.0f;
  const int nblk = sg.n_out / 32;
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int orow = row0 + 16 * r + 4 * g4 + i;
      float v[NT / 2];
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < half; ++j) {
        v[j] = situ_f(acc[r][j][i], acc[r][j + half][i], g.beta, inv_b, g.lbeta, inv_lb);
        amax = fmaxf(amax, fabsf(v[j]));
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, WAVE));
      const int X = mx_e4m3_exponent(amax);
      if (pair_o[r][i] < 0) continue;
      uint8_t* act = reinterpret_cast<uint8_t*>(sg.out) + (size_t)orow * sg.ldo;
#pragma unroll
      for (int j = 0; j < half; ++j) act[nb * half * 16 + j * 16 + m] = (uint8_t)e4m3_encode(__builtin_ldexpf(v[j], -X));
      if (m == 0) g.out_scale[(size_t)orow * nblk + nb] = (uint8_t)(X + 127);
    }
  }
}

// ---- FC2 with the activation tile in LDS (32-row tiles, K = d = 512) -----------------
// The 4 wavefronts of a workgroup share one 32-row tile and walk MX_FC2_BLOCKS_PER_WAVE
// neighbouring column blocks each. The tile's activation codes (32 x 512 e4m3 bytes) and
// scales (32 x 16 bytes) are copied into LDS once, by buffer-to-LDS copies, before the
// walk; the wavefronts read their fragments from there and load only the weights. Chunk c
// (16 bytes) of row j sits at position c ^ (j % 16) of the row's 512 bytes, so that the
// 16 rows one read instruction touches fall into 16 different bank groups; the positions
// of the second 256-wide K step are those of the first plus 256 bytes.
constexpr int MXF2_A = 32 * 512;                  // activation codes of the tile
constexpr int MXF2_LDS = MXF2_A + 32 * 16;        // + their scales

template <int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void mx_fc2_lds_kernel(
    const StreamGemm g, int blocks_total, int wgs_per_tile) {
  __shared__ __attribute__((aligned(1024))) char smem[MXF2_LDS];
  constexpr int R = 2, BPW = MX_FC2_BLOCKS_PER_WAVE, NSTEP = 2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mt = (int)blockIdx.x / wgs_per_tile;
  const int nb0 = ((int)blockIdx.x - mt * wgs_per_tile) * 4 * BPW + wave * BPW;   // first block of this wave
  const int row0 = mt * 32;
  if (row0 >= g.M) return;
  const int e = __builtin_amdgcn_readfirstlane(g.tile_expert[row0 / g.tile_m]);
  if (e < 0) return;
  const int first = __builtin_amdgcn_readfirstlane(g.row_to_pair[row0]);
  if (first < 0) return;
  const Seg sg = g.seg[0];
  const int m = lane & 15, g4 = lane >> 4;
  const int Kd = g.Kd;            // 512
  const int nst = Kd / 512;       // 1

  // every row id this wavefront needs, requested together before any is used: the output
  // rows' pairs, the rows its activation copies read (4 of codes, 2 of scales)
  int pair_o[R][4], cp_row[4], sc_row[2];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) pair_o[r][i] = g.row_to_pair[row0 + 16 * r + 4 * g4 + i];
#pragma unroll
  for (int i = 0; i < 4; ++i) cp_row[i] = g.row_to_pair[row0 + 2 * (4 * wave + i) + (lane >> 5)];
#pragma unroll
  for (int k = 0; k < 2; ++k) sc_row[k] = g.row_to_pair[row0 + ((256 * k + 4 * lane) >> 4)];

  // ---- the tile's activation rows into LDS: copy i (4 per wavefront) covers rows 2 i',
  // 2 i' + 1 (i' = 4 wave + i), the lane filling position lane % 32 of row 2 i' + lane / 32
  // with chunk (lane % 32) ^ (row % 16); every wavefront copies all 512 scale bytes (two
  // copies of 64 lanes x 4 bytes: lane -> row (256 k + 4 lane) / 16)
  const rsrc_t ac_rs = make_rsrc(uniform_ptr(g.a), __builtin_amdgcn_readfirstlane(g.a_bytes));
  const rsrc_t as_rs = make_rsrc(uniform_ptr(g.a_scale), __builtin_amdgcn_readfirstlane(g.a_scale_bytes));
  // FC2 reads the permuted rows themselves; a pad row reads the tile's first
  auto a_row = [&](int j, int p) { return p >= 0 ? row0 + j : row0; };
  uint32_t cp_off[4], sc_off[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 2 * (4 * wave + i) + (lane >> 5);
    cp_off[i] = (uint32_t)a_row(j, cp_row[i]) * (uint32_t)Kd + (uint32_t)(((lane & 31) ^ (j & 15)) * 16);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int byte = 256 * k + 4 * lane;          // of the 512: row byte / 16, offset byte % 16
    sc_off[k] = (uint32_t)a_row(byte >> 4, sc_row[k]) * (uint32_t)(Kd / 32) + (uint32_t)(byte & 15);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) to_lds(ac_rs, smem + (4 * wave + i) * 1024, cp_off[i], 0);
#pragma unroll
  for (int k = 0; k < 2; ++k)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(as_rs, (lds_void*)(smem + MXF2_A + 256 * k), 4, sc_off[k], 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  // combine weights of the output rows (their latency hides behind the copies)
  float pw[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) pw[r][i] = (g.pair_w != nullptr && pair_o[r][i] >= 0) ? g.pair_w[pair_o[r][i]] : 1.0f;

  // ---- weights: block bi of the walk, step s (K 256 s ..), as in the register-only kernel
  const uint32_t wc_bytes = __builtin_amdgcn_readfirstlane((uint32_t)sg.n_total * (uint32_t)(Kd / 2));
  const uint32_t ws_bytes = __builtin_amdgcn_readfirstlane((uint32_t)sg.n_total * (uint32_t)(Kd / 32));
  const rsrc_t wc_rs = make_rsrc(uniform_ptr(reinterpret_cast<const uint8_t*>(sg.w) + (size_t)e * wc_bytes), wc_bytes);
  const rsrc_t ws_rs = make_rsrc(uniform_ptr(g.w_scale + (size_t)e * ws_bytes), ws_bytes);
  const int nblk_w = max(0, min(BPW, blocks_total - nb0));   // blocks this wavefront stores
  auto load_b = [&](int t, MxB<NT>& st) __attribute__((always_inline)) {
    const int tc = min(t, BPW * NSTEP - 1);
    const int bi = min(tc >> 1, max(nblk_w - 1, 0));
    const int h = tc & 1;
    const uint32_t nbase = (uint32_t)(min(nb0 + bi, blocks_total - 1) * NT);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = 2 * h + u;
#pragma unroll
      for (int j = 0; j < NT; ++j)
        st.b[j][u] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(wc_rs, lane * 16, ((nbase + j) * nst) * 4096u + q * 1024u, 0));
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) st.sb[j] = __builtin_amdgcn_raw_buffer_load_b32(ws_rs, lane * 4, ((nbase + j) * nst) * 256u, 0);
  };
  MxB<NT> b0, b1;
  load_b(0, b0);
  __builtin_amdgcn_sched_barrier(0);
  // this wavefront's copies are done once only the 12 weight loads after them may be
  // outstanding; then every wavefront's
  __builtin_amdgcn_s_waitcnt(waitcnt(12, 15));
  lds_barrier();

  // fragment addresses of step 0 (step 1: + 256 bytes of codes, + 8 bytes of scales)
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  uint32_t ra[R][2][2], rs[R][2];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int v = 0; v < 2; ++v)
        ra[r][u][v] = lds_base + (uint32_t)((16 * r + m) * 512 + (((8 * u + 4 * v + g4) ^ m) * 16));
      rs[r][u] = lds_base + (uint32_t)(MXF2_A + (16 * r + m) * 16 + 4 * u + g4);
    }
  auto read_a = [&ra, &rs](auto S, mx_u32x4 (&a)[R][2][2], uint32_t (&sa)[R][2]) __attribute__((always_inline)) {
    constexpr int OA = decltype(S)::value * 256, OS = decltype(S)::value * 8;
    asm volatile(
        "ds_read_b128 %0, %12 offset:%24\n"
        "ds_read_b128 %1, %13 offset:%24\n"
        "ds_read_b128 %2, %14 offset:%24\n"
        "ds_read_b128 %3, %15 offset:%24\n"
        "ds_read_b128 %4, %16 offset:%24\n"
        "ds_read_b128 %5, %17 offset:%24\n"
        "ds_read_b128 %6, %18 offset:%24\n"
        "ds_read_b128 %7, %19 offset:%24\n"
        "ds_read_u8 %8, %20 offset:%25\n"
        "ds_read_u8 %9, %21 offset:%25\n"
        "ds_read_u8 %10, %22 offset:%25\n"
        "ds_read_u8 %11, %23 offset:%25\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0][0][0]), "=&v"(a[0][0][1]), "=&v"(a[0][1][0]), "=&v"(a[0][1][1]), "=&v"(a[1][0][0]),
          "=&v"(a[1][0][1]), "=&v"(a[1][1][0]), "=&v"(a[1][1][1]), "=&v"(sa[0][0]), "=&v"(sa[0][1]),
          "=&v"(sa[1][0]), "=&v"(sa[1][1])
        : "v"(ra[0][0][0]), "v"(ra[0][0][1]), "v"(ra[0][1][0]), "v"(ra[0][1][1]), "v"(ra[1][0][0]),
          "v"(ra[1][0][1]), "v"(ra[1][1][0]), "v"(ra[1][1][1]), "v"(rs[0][0]), "v"(rs[0][1]), "v"(rs[1][0]),
          "v"(rs[1][1]), "i"(OA), "i"(OS)
        : "memory");
  };

  floatx4 acc[R][NT];
  auto zero = [&]() {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[r][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  };
  zero();
  auto consume = [&](int h, const mx_u32x4 (&a)[R][2][2], const uint32_t (&sa)[R][2], const MxB<NT>& st)
      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const intx8 av = {(int)a[r][u][0][0], (int)a[r][u][0][1], (int)a[r][u][0][2], (int)a[r][u][0][3],
                          (int)a[r][u][1][0], (int)a[r][u][1][1], (int)a[r][u][1][2], (int)a[r][u][1][3]};
        const int sav = (int)(sa[r][u] & 0xFFu);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const intx8 bv = {(int)st.b[j][u].x, (int)st.b[j][u].y, (int)st.b[j][u].z, (int)st.b[j][u].w, 0, 0, 0, 0};
          const int sb = (int)((st.sb[j] >> (8 * (2 * h + u))) & 0xFFu);
          acc[r][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[r][j], 0, 4, 0, sav, 0, sb);
        }
      }
    }
  };
  // weighted per-pair products (or the token row when K = 1) of column block nbc
  auto store = [&](int nbc) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < R; ++r)
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
          else if (sg.out_elt == Elt::F32)
            reinterpret_cast<float*>(sg.out)[(size_t)(pair / g.topk) * sg.ldo + col] = wgt * acc[r][j][i];
          else
            reinterpret_cast<uint16_t*>(sg.out)[(size_t)(pair / g.topk) * sg.ldo + col] = f32_to_bf16(wgt * acc[r][j][i]);
        }
      }
  };
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  // the walk, unrolled: block bi = t / 2, K step t % 2; the next step's weights load while
  // this one computes (and while the last block's products are stored)
  static_for<BPW>([&](auto BI) __attribute__((always_inline)) {
    constexpr int bi = decltype(BI)::value;
    mx_u32x4 a[R][2][2];
    uint32_t sa[R][2];
    read_a(H0{}, a, sa);
    load_b(2 * bi + 1, b1);
    __builtin_amdgcn_sched_barrier(0);
    consume(0, a, sa, b0);
    read_a(H1{}, a, sa);
    load_b(2 * bi + 2, b0);
    __builtin_amdgcn_sched_barrier(0);
    consume(1, a, sa, b1);
    if (bi < nblk_w) store(nb0 + bi);
    zero();
  });
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
      hipLaunchKernelGGL((mx_fc1_lds_kernel<NT>), dim3(grid), dim3(threads), 0, stream, g, blocks, nsteps);
    else
      hipLaunchKernelGGL((stream_gemm_mx_kernel<NT, 1>), dim3(grid), dim3(threads), 0, stream, g, blocks, nsteps, 1);
  } else if (R == 2 && g.Kd == 512) {
    // 4 wavefronts per workgroup on one tile, MX_FC2_BLOCKS_PER_WAVE blocks each
    const int wpt = (blocks + 4 * bpw - 1) / (4 * bpw);
    hipLaunchKernelGGL((mx_fc2_lds_kernel<NT>), dim3((unsigned)(m_tiles * wpt)), dim3(256), 0, stream, g, blocks, wpt);
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
