// LDS-tiled MFMA GEMM for gfx950 (bf16 in, fp32 accumulate) for the token-heavy calls:
// the prefill-sized projections of the hidden input, the tail, and the grouped expert
// FC1 / FC2 over tiles of 128 expert rows.
//
// Workgroup tile: 128 rows x 512 weight rows, 512 threads = 8 wavefronts, two per SIMD:
// wavefront w owns rows 64 (w / 4) .. + 63 x weight rows 128 (w % 4) .. + 127 as 2 x 4
// v_mfma_f32_32x32x16_bf16 tiles (128 fp32 accumulators per lane). With two wavefronts per
// SIMD, one's waits (for a buffer-to-LDS copy to be taken, for LDS) overlap the other's
// MFMAs; against four wavefronts of 256 accumulators the epilogue halves and the K loop
// stays where it was, held by the rate at which a CU pulls operands into LDS (40 KB per
// step in about 1800 cycles). A SituGLU column block holds 64 gate rows and the matching
// 64 up rows. Per 32-wide K step the workgroup needs 8 KB of activations and 32 KB of
// weights for 1024 MFMA cycles per SIMD, and each wavefront reads 12 KB of operands from
// LDS.
//
// Operands reach LDS by direct buffer-to-LDS loads (buffer_load_dwordx4 ... lds) in the
// packed MFMA order the weights already have in HBM: for each 16-row group and 32-wide K
// step, a 1 KB block holding lane l = 16g + r's 16 bytes (row r, K 8g .. 8g + 7) at 16 l.
// A 32 x 32 x 16 operand (row l % 32, K 8 (l / 32) .. + 7 of one half step) is then one
// conflict-free ds_read_b128 from two neighbouring blocks, and the weights are copied
// block for block; each wavefront copies one activation block and four weight blocks per
// step. LDS is a ring of NSLOT 40 KB K steps, NSLOT - 1 of them in flight while one is
// computed; the operands of step c + 1 are read from LDS into registers while the MFMAs of
// step c run. Groups of 8 row tiles x all weight blocks share their operands in one XCD's
// L2.
//
// A wavefront computes only those of its two 32-row tiles that hold a row to store: the
// padding at the end of an expert's last tile (and, in the dense launches that need no
// tail or add, rows past M) takes no MFMAs and no fragment reads, while the copies, waits
// and barriers stay those of every other wavefront (the copy lanes of such rows read past
// the end of the buffer, which costs no memory request).
//
// The epilogue goes through LDS 32 rows per wavefront at a time; the pair ids of the
// tile's rows are requested before the K loop and the combine weights and in-place
// addends before the stores, so that no output row waits on a dependent global load.
//
// Epilogues: plain store, SituGLU (vLLM PR 50088, commit 2), weighted per-pair store for
// the combine (TensorRT-LLM PR 20541, "Commit 1": finalize), and the in-place add of the
// up projection (vLLM latent_moe_runner page, _shard_up_proj_tail).
#include "common.h"
#include "kernels.h"

namespace lmoe {

constexpr int TILE_M = 128;
constexpr int TILE_N = 512;           // weight rows per workgroup (SituGLU: 256 gate + 256 up)
constexpr int NSLOT = 4;              // LDS ring of K steps
constexpr int SLOT = 40960;           // bytes per K step: A 8 x 1 KB + B 32 x 1 KB
constexpr int B_OFF = 8192;
constexpr int LOADS_PER_STEP = 5;     // per wavefront: 1 A block + 4 B blocks
constexpr int GROUP_M = 8;            // row tiles per swizzle group

// four consecutive outputs as fp32 (16 bytes) or bf16 (8 bytes)
LMOE_DEV void store4(Elt elt, void* base, size_t idx, floatx4 v) {
  if (elt == Elt::F32) {
    *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(base) + idx) = v;
  } else {
    const uint32_t lo = pack_bf16x2(v[0], v[1]);
    const uint32_t hi = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + idx) = make_uint2(lo, hi);
  }
}

// 16-byte LDS read at byte address addr + OFF. Issued as inline assembly: the compiler
// would otherwise wait for every outstanding buffer-to-LDS load before any LDS read (it
// cannot tell which LDS bytes they write). The caller waits (lgkmcnt) before using the
// result; in this kernel every step starts with s_waitcnt lgkmcnt(0) and a barrier, and
// fragments are used one step after they are read.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
template <int OFF>
LMOE_DEV bf16x8_t lds_read16(uint32_t addr) {
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return __builtin_bit_cast(bf16x8_t, r);
}

struct Frag {
  bf16x8_t a[4], b[8];
};

template <bool ADD_PRE, bool DUAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void tiled_gemm_kernel(
    const StreamGemm g, int blocks_total, int m_tiles, int nch_total) {
  __shared__ __attribute__((aligned(1024))) char smem[NSLOT * SLOT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 0 .. 7
  const int cb = wave & 3;     // the wavefront's 128 weight rows (column block of the tile)
  const int rh = wave >> 2;    // the wavefront's 64 rows of the tile
  const int m = lane & 15, g4 = lane >> 4;

  // ---- tile of this workgroup. Logical ids come in groups of GROUP_M row tiles x all
  // weight blocks (one group shares its operands in one L2; workgroup b runs on XCD
  // b % 8). Dense launches give each XCD an equal run of consecutive ids. Grouped launches
  // deal whole groups to the XCDs in turn: their tiles that hold rows come first, and the
  // rest return at once, so equal runs would leave the last XCDs idle. With split-K the K
  // slice is the outermost index.
  const int G = m_tiles * blocks_total;
  const int ksplit = g.ksplit > 1 ? g.ksplit : 1;
  const int per_group = GROUP_M * blocks_total;
  const int j = (int)(blockIdx.x >> 3);
  const int lid_k = g.row_to_pair != nullptr
                        ? ((j / per_group) * 8 + (int)(blockIdx.x & 7)) * per_group + j % per_group
                        : (int)(blockIdx.x & 7) * (int)(gridDim.x >> 3) + j;
  if (lid_k >= G * ksplit) return;
  const int ks = lid_k / G;
  const int lid = lid_k - ks * G;
  const int k0 = (int)((long)nch_total * ks / ksplit);                 // this slice's K steps
  const int nch = (int)((long)nch_total * (ks + 1) / ksplit) - k0;
  const int grp = lid / per_group;
  const int first_m = grp * GROUP_M;
  const int gm = min(GROUP_M, m_tiles - first_m);
  const int within = lid - grp * per_group;
  const int mt = first_m + within % gm;
  const int nb_all = within / gm;
  const int row0 = mt * TILE_M;

  int s = 0;
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (i < g.nseg && nb_all >= g.seg[i].block0) s = i;
  const Seg sg = g.seg[s];
  const int nb = nb_all - sg.block0;
  const bool situ = sg.epi == Epi::SITU;
  const bool grouped = g.row_to_pair != nullptr;
  int e = 0;
  if (grouped) {
    e = __builtin_amdgcn_readfirstlane(g.tile_expert[row0 / g.tile_m]);
    if (e < 0) return;
  }

  // ---- activation rows this wavefront copies (row group `wave` of the tile's 8)
  rsrc_t a_rs = make_rsrc(uniform_ptr(g.a), __builtin_amdgcn_readfirstlane(g.a_bytes));
  uint32_t a_off;
  {
    const int row = row0 + 16 * wave + m;
    // Padding rows (and rows past M) copy from past the end of the buffer: the hardware
    // range check turns those lanes' copies into zeros without a memory request (their
    // products are never stored). Buffers within 1 MB of 4 GB copy row 0 instead.
    int arow;
    if (grouped) {
      const int p = g.row_to_pair[row];
      arow = p >= 0 ? (g.a_by_row ? row : p / g.topk) : -1;
    } else {
      arow = row < g.M ? row : -1;
    }
    const uint32_t pad_off = g.a_bytes <= 0xFFF00000u ? g.a_bytes : 0u;
    a_off = (arow >= 0 ? (uint32_t)arow * (uint32_t)(g.lda * 2) : pad_off) + g4 * 16;
  }
  // pair of the output row row0 + 64 rh + lane (-1: padding or past M), read by the
  // epilogue; requested here so that its latency hides behind the K loop
  int rp;
  {
    const int row = row0 + 64 * rh + lane;
    rp = grouped ? g.row_to_pair[row] : (row < g.M ? row : -1);
  }

  // ---- weight row groups this wavefront copies: LDS blocks 4 wave .. 4 wave + 3 of the
  // 32 (block q holds row group q % 8 of column block q / 8; SituGLU: 4 gate + 4 up)
  const uint32_t w_bytes = __builtin_amdgcn_readfirstlane((uint32_t)sg.n_total * (uint32_t)(g.Kd * 2));
  rsrc_t w_rs = make_rsrc(uniform_ptr(reinterpret_cast<const char*>(sg.w) + (size_t)e * w_bytes), w_bytes);
  auto n16_of = [&](int q) __attribute__((always_inline)) {
    const int cw = q >> 3, j = q & 7;
    return situ ? (j < 4 ? nb * 16 + 4 * cw + j : sg.n_out / 16 + nb * 16 + 4 * cw + (j - 4))
                : nb * 32 + 8 * cw + j;
  };
  uint32_t b_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    b_off[j] = (uint32_t)n16_of(4 * wave + j) * (uint32_t)(g.Kd * 32) + lane * 16;   // past the matrix: zeros

  // Two K phases (DUAL, dense, one plain segment): steps 0 .. nch0 - 1 multiply `a` by the
  // segment's weights, the rest `a1` by `w1`, accumulating into the same fp32 tiles, so
  // that the result is round(a w^T + a1 w1^T). The copies run ahead of the MFMAs, so the
  // operands switch when the first copy of step nch0 is issued.
  const int nch0 = DUAL ? g.Kd / 32 : nch_total;
  int kb = 0;                              // first step of the phase being copied
  auto to_phase1 = [&]() __attribute__((always_inline)) {
    a_rs = make_rsrc(uniform_ptr(g.a1), __builtin_amdgcn_readfirstlane(g.a1_bytes));
    a_off = (uint32_t)min(row0 + 16 * wave + m, g.M - 1) * (uint32_t)(g.lda1 * 2) + g4 * 16;
    const uint32_t w1_bytes = __builtin_amdgcn_readfirstlane((uint32_t)sg.n_total * (uint32_t)(g.Kd1 * 2));
    w_rs = make_rsrc(uniform_ptr(g.w1), w1_bytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) b_off[j] = (uint32_t)n16_of(4 * wave + j) * (uint32_t)(g.Kd1 * 32) + lane * 16;
    kb = nch0;
  };
  // a split-K slice that starts in the second phase copies its operands from the start
  if constexpr (DUAL)
    if (k0 >= nch0) to_phase1();
  // copy k of step c: k = 0 this wavefront's activation row group, 1 .. 4 its four weight
  // row groups
  auto issue_one = [&](int c, int k) __attribute__((always_inline)) {
    char* base = smem + (c % NSLOT) * SLOT;
    if (k < 1)
      to_lds(a_rs, base + wave * 1024, a_off, (uint32_t)(c + k0 - kb) * 64u);
    else
      to_lds(w_rs, base + B_OFF + (4 * wave + k - 1) * 1024, b_off[k - 1], (uint32_t)(c + k0 - kb) * 1024u);
  };
  auto issue = [&](int c) {
    if constexpr (DUAL)
      if (c + k0 == nch0) to_phase1();
#pragma unroll
    for (int k = 0; k < LOADS_PER_STEP; ++k) issue_one(c, k);
  };
  // 32 x 32 x 16 operand of lane l: row l % 32 of a 32-row tile (16-row block (l / 16) & 1),
  // K 8 (l / 32) .. + 7 of the half step h: K group 2 h + l / 32 of that block
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)smem + ((lane >> 4) & 1) * 1024 + (lane >> 5) * 256 + (lane & 15) * 16;
  // fragment K (a compile-time 0 .. 11) of step c: 0 .. 3 activation tile K / 2 of the
  // wavefront's two (32-row tiles 2 rh, 2 rh + 1), half step K % 2; 4 .. 11 weight tile
  // (K - 4) / 2 of its column block, half step K % 2
  const uint32_t lds_a = lds0 + (uint32_t)rh * 4096;
  const uint32_t lds_b = lds0 + B_OFF + (uint32_t)cb * 8192;
  // NA (compile time): how many of the wavefront's two 32-row tiles it computes; the
  // fragments of the others are not read
  auto read_one = [&](int c, Frag& f, auto K, auto NA) __attribute__((always_inline)) {
    constexpr int k = decltype(K)::value;
    constexpr int na = decltype(NA)::value;
    if constexpr (k < 4) {
      if constexpr ((k >> 1) < na)
        f.a[k] = lds_read16<(k >> 1) * 2048 + (k & 1) * 512>(lds_a + (uint32_t)(c % NSLOT) * SLOT);
    } else if constexpr (na > 0) {
      constexpr int q = k - 4;
      f.b[q] = lds_read16<(q >> 1) * 2048 + (q & 1) * 512>(lds_b + (uint32_t)(c % NSLOT) * SLOT);
    }
  };
  auto read = [&](int c, Frag& f, auto NA) { static_for<12>([&](auto k) { read_one(c, f, k, NA); }); };

  floatx16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};

  auto mma = [&](const Frag& f, auto NA) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < decltype(NA)::value; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[2 * i + h], f.b[2 * j + h], acc[i][j], 0, 0, 0);
  };

  // ---- prologue: steps 0 .. NSLOT-1 in flight; step 0 in registers
#pragma unroll
  for (int c = 0; c < NSLOT; ++c)
    if (c < nch) issue(c);
  // wait until at most `ahead` later steps of this wavefront are still in flight
  auto wait_steps = [&](int ahead) {
    if (ahead >= 3)
      __builtin_amdgcn_s_waitcnt(waitcnt(3 * LOADS_PER_STEP, 0));
    else if (ahead == 2)
      __builtin_amdgcn_s_waitcnt(waitcnt(2 * LOADS_PER_STEP, 0));
    else if (ahead == 1)
      __builtin_amdgcn_s_waitcnt(waitcnt(LOADS_PER_STEP, 0));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
  };
  wait_steps(min(nch, NSLOT) - 1);
  lds_barrier();
  // The wavefront's 32-row tiles that hold a row to store (padding rows and rows past M
  // come last in a tile): only those are computed, and a wavefront with none only copies.
  // Its row ids were requested before the copies, so they have landed by now.
  const uint64_t mv = __ballot(rp >= 0);
  const int nv = mv ? 64 - __builtin_clzll(mv) : 0;
  const int n_act = __builtin_amdgcn_readfirstlane((nv + 31) >> 5);

  // ---- main loop, two steps per trip so that the register fragments alternate.
  // Step c: wait until step c + 1 has landed (this wavefront's loads, then the barrier for
  // the others) and this wavefront's reads of step c (slot c % NSLOT) are done; after the
  // barrier every wavefront is done with that slot, and step c + NSLOT goes into it. Then
  // read step c + 1 into registers while the MFMAs of step c run.
  auto step = [&](int c, Frag& cur, Frag& nxt, auto NA) {
    // issued so far: steps up to min(c + NSLOT - 1, nch - 1)
    wait_steps(min(c + NSLOT - 1, nch - 1) - (c + 1));
    lds_barrier();                        // nothing moves across the waits and the barrier
    // fragment reads, then the MFMAs, then the copies of step c + NSLOT: a wavefront's
    // buffer-to-LDS copies can hold up its in-order issue (measured: placed before the
    // MFMAs they cost about 3% more per step than placed after them)
    if (c + 1 < nch) read(c + 1, nxt, NA);
    mma(cur, NA);
    __builtin_amdgcn_sched_barrier(0);
    if (c + NSLOT < nch) issue(c + NSLOT);
  };
  // Steps whose copy c + NSLOT exists: the fragment reads follow the first 12 MFMAs one by
  // one and the 5 copies every third MFMA, each pinned in place, so that a wait for the
  // address unit to take a copy overlaps the MFMA already running (and the other
  // wavefront of the SIMD).
  auto step_il = [&](int c, Frag& cur, Frag& nxt, auto NA) __attribute__((always_inline)) {
    wait_steps(NSLOT - 2);
    lds_barrier();
    if constexpr (DUAL)
      if (c + NSLOT + k0 == nch0) to_phase1();
    static_for<16>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      constexpr int h = i >> 3, ti = (i >> 2) & 1, tj = i & 3;
      if constexpr (ti < decltype(NA)::value)
        acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[2 * ti + h], cur.b[2 * tj + h], acc[ti][tj], 0, 0, 0);
      if constexpr (i < 12) read_one(c + 1, nxt, std::integral_constant<int, i>{}, NA);
      if constexpr (i % 3 == 1 && i / 3 < LOADS_PER_STEP) issue_one(c + NSLOT, i / 3);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto k_loop = [&](auto NA) __attribute__((always_inline)) {
    Frag f0, f1;
    read(0, f0, NA);
    int c = 0;
    for (; c + 1 + NSLOT < nch; c += 2) {
      step_il(c, f0, f1, NA);
      step_il(c + 1, f1, f0, NA);
    }
    for (; c + 1 < nch; c += 2) {
      step(c, f0, f1, NA);
      step(c + 1, f1, f0, NA);
    }
    if (c < nch) step(c, f0, f1, NA);
  };
  // (the dense-only variants, the tail and the in-place add, compute every tile: only
  // their last row tile can hold rows past M)
  if (DUAL || ADD_PRE || n_act == 2)
    k_loop(std::integral_constant<int, 2>{});
  else if (n_act == 1)
    k_loop(std::integral_constant<int, 1>{});
  else
    k_loop(std::integral_constant<int, 0>{});

  // ---- epilogue, 32 rows at a time through this wavefront's own LDS region (every
  // wavefront is past its last LDS read and every buffer-to-LDS load has landed): the
  // accumulators of 32 rows are written to LDS as fp32 [32][RS], then read back as 4
  // consecutive columns per lane so that the outputs leave as contiguous row segments.
  constexpr int RS = 132;                          // row stride (floats), padded against bank conflicts
  float* red = reinterpret_cast<float*>(smem) + wave * (32 * RS);
  const float inv_b = 1.0f / g.beta;
  const float inv_lb = g.lbeta > 0.0f ? 1.0f / g.lbeta : 0.0f;
  // combine weight of this lane's row, requested once for the whole epilogue
  float rw = 1.0f;
  if ((sg.epi == Epi::PAIR || sg.epi == Epi::TOKEN) && g.pair_w) rw = rp >= 0 ? g.pair_w[rp] : 0.0f;
  // rows of the wavefront's 64 up to the last one holding a pair (nv, dense: the last one
  // below M); the loops below skip whole batches of rows past it
  const int nvq[2] = {min(nv, 32), max(nv - 32, 0)};
  const int rbase0 = row0 + 64 * rh;
  // accumulator tile (t, j) register rr: row 8 (rr / 4) + 4 (lane / 32) + rr % 4 of the
  // wavefront's 32-row tile t, column 32 j + lane % 32 of its 128 columns
  auto acc_to_lds = [&](auto T) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    static_for<4>([&](auto j) {
      static_for<16>([&](auto rr) {
        red[(8 * (int(rr) >> 2) + 4 * (lane >> 5) + (int(rr) & 3)) * RS + 32 * j + (lane & 31)] =
            acc[int(T)][int(j)][int(rr)];
      });
    });
    __builtin_amdgcn_sched_barrier(0);
  };

  if (ksplit > 1) {
    // raw fp32 partial sums of this K slice: 32 lanes per row, 4 weight-row columns each
    int pbase = 0, ptot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < g.nseg) {
        if (i < s) pbase += g.seg[i].n_total;
        ptot += g.seg[i].n_total;
      }
    }
    const int q = lane & 31;
    int pcol, valid;
    if (situ) {
      const int c = 4 * q;   // LDS columns 0..63: gate, 64..127: up
      const int oc = 256 * nb + 64 * cb + (c & 63);
      valid = oc < sg.n_out;
      pcol = (c < 64 ? 0 : sg.n_out) + oc;
    } else {
      pcol = TILE_N * nb + 128 * cb + 4 * q;
      valid = pcol < sg.n_out;
    }
    float* dst = g.part + (size_t)ks * g.M * ptot + pbase + pcol;
    static_for<2>([&](auto t) {
      acc_to_lds(t);
      const int rbase = rbase0 + 32 * int(t);
      for (int r = lane >> 5; r < 32; r += 2) {
        const int row = rbase + r;
        const floatx4 v = *reinterpret_cast<const floatx4*>(red + r * RS + 4 * q);
        if (row < g.M && valid) *reinterpret_cast<floatx4*>(dst + (size_t)row * ptot) = v;
      }
    });
    return;
  }

  // The output loops, specialised on the epilogue and the output type (both uniform in a
  // workgroup) so that they hold no per-row branches on them: in each batch of rows, the
  // LDS reads, row ids and combine weights are all requested before the first store, so
  // that no read waits behind a store or a branch; batches past the last row holding a
  // pair are skipped. The loop over the two 32-row tiles is not unrolled: the epilogue runs
  // once per workgroup, so its code is fetched cold, and a compact loop keeps that short.
  auto epilogue = [&](auto EP, auto F32OUT) __attribute__((always_inline)) {
    constexpr Epi ep = decltype(EP)::value;
    constexpr Elt oe = decltype(F32OUT)::value ? Elt::F32 : Elt::BF16;
    constexpr bool add_pre = ep == Epi::ADD && oe == Elt::BF16;
#pragma unroll 1
    for (int t = 0; t < 2; ++t) {
      const int nvt = t ? nvq[1] : nvq[0];
      if (nvt == 0) break;
      const int rbase = rbase0 + 32 * t;
      // in-place addends (bf16) of every row of this tile that this lane stores, requested
      // before its stores: vector-memory stores and loads share one in-order counter, so a
      // load issued after a store would wait for it (each element is read and written by
      // the same lane, so `add` may be the output)
      [[maybe_unused]] uint2 addv[add_pre ? 2 : 1][8];
      if constexpr (add_pre) {
        const int col = TILE_N * nb + 128 * cb + 4 * (lane & 31);
#pragma unroll
        for (int bt = 0; bt < 2; ++bt)
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int r = 16 * bt + 2 * u + (lane >> 5);
            addv[bt][u] = make_uint2(0u, 0u);
            if (g.add != nullptr && r < nvt && rbase + r < g.M && col < sg.n_out)
              addv[bt][u] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(g.add) +
                                                            (size_t)(rbase + r) * sg.ldo + col);
          }
      }
      if (t == 0)
        acc_to_lds(std::integral_constant<int, 0>{});
      else
        acc_to_lds(std::integral_constant<int, 1>{});
      if constexpr (ep == Epi::SITU) {
        // 16 lanes per row (4 outputs each): gate columns c .. c + 3, up columns 64 + c ..;
        // one batch of 32 rows, 8 per lane
        const int q = lane & 15;
        const int col = 256 * nb + 64 * cb + 4 * q;
        const bool col_ok = col < sg.n_out;
        floatx4 gv[8], uv[8];
        int pr[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = 4 * u + (lane >> 4);
          pr[u] = __shfl(rp, 32 * t + r, WAVE);
          gv[u] = *reinterpret_cast<const floatx4*>(red + r * RS + 4 * q);
          uv[u] = *reinterpret_cast<const floatx4*>(red + r * RS + 64 + 4 * q);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (pr[u] < 0 || !col_ok) continue;
          floatx4 v;
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = situ_f(gv[u][k], uv[u][k], g.beta, inv_b, g.lbeta, inv_lb);
          store4(oe, sg.out, (size_t)(rbase + 4 * u + (lane >> 4)) * sg.ldo + col, v);
        }
      } else {
        // 32 lanes per row (4 columns each), batches of 16 rows, 8 per lane
        const int q = lane & 31;
        const int col = TILE_N * nb + 128 * cb + 4 * q;
        const bool col_ok = col < sg.n_out;
        auto batch = [&](int r0, auto BT) __attribute__((always_inline)) {
          floatx4 v[8];
          int pr[8];
          [[maybe_unused]] float wt[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int r = r0 + 2 * u + (lane >> 5);
            pr[u] = __shfl(rp, 32 * t + r, WAVE);
            if constexpr (ep == Epi::PAIR || ep == Epi::TOKEN) wt[u] = __shfl(rw, 32 * t + r, WAVE);
            v[u] = *reinterpret_cast<const floatx4*>(red + r * RS + 4 * q);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            if (pr[u] < 0 || !col_ok) continue;
            const size_t idx = (size_t)(rbase + r0 + 2 * u + (lane >> 5)) * sg.ldo + col;
            if constexpr (ep == Epi::PAIR) {
              // non-temporal: the products are read back once, by the combine, after the
              // rest of the launch has passed through the caches (measured 5% faster)
              __builtin_nontemporal_store(
                  v[u] * wt[u], reinterpret_cast<floatx4*>(reinterpret_cast<float*>(sg.out) + (size_t)pr[u] * sg.ldo + col));
            } else if constexpr (ep == Epi::TOKEN) {
              store4(oe, sg.out, (size_t)(pr[u] / g.topk) * sg.ldo + col, v[u] * wt[u]);
            } else if constexpr (ep == Epi::ADD) {
              if constexpr (add_pre) {
                const uint2 a = addv[decltype(BT)::value][u];
                v[u] += floatx4{__uint_as_float(a.x << 16), __uint_as_float(a.x & 0xFFFF0000u),
                                __uint_as_float(a.y << 16), __uint_as_float(a.y & 0xFFFF0000u)};
              } else if (g.add != nullptr) {
                v[u] += *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(g.add) + idx);
              }
              store4(oe, sg.out, idx, v[u]);
            } else {
              store4(oe, sg.out, idx, v[u]);
            }
          }
        };
        if constexpr (add_pre) {
          // the addends sit in registers per batch: batches unrolled
          static_for<2>([&](auto bt) {
            if (16 * int(bt) < nvt) batch(16 * int(bt), bt);
          });
        } else {
#pragma unroll 1
          for (int r0 = 0; r0 < nvt; r0 += 16) batch(r0, std::integral_constant<int, 0>{});
        }
      }
    }
  };
  using F32_ = std::true_type;
  using BF16_ = std::false_type;
  const bool f32out = sg.out_elt == Elt::F32;
  if constexpr (ADD_PRE) {
    epilogue(std::integral_constant<Epi, Epi::ADD>{}, BF16_{});
  } else if constexpr (DUAL) {
    if (f32out)
      epilogue(std::integral_constant<Epi, Epi::STORE>{}, F32_{});
    else
      epilogue(std::integral_constant<Epi, Epi::STORE>{}, BF16_{});
  } else if (sg.epi == Epi::SITU) {
    if (f32out)
      epilogue(std::integral_constant<Epi, Epi::SITU>{}, F32_{});
    else
      epilogue(std::integral_constant<Epi, Epi::SITU>{}, BF16_{});
  } else if (sg.epi == Epi::PAIR) {
    epilogue(std::integral_constant<Epi, Epi::PAIR>{}, F32_{});
  } else if (sg.epi == Epi::TOKEN) {
    if (f32out)
      epilogue(std::integral_constant<Epi, Epi::TOKEN>{}, F32_{});
    else
      epilogue(std::integral_constant<Epi, Epi::TOKEN>{}, BF16_{});
  } else if (sg.epi == Epi::ADD) {
    epilogue(std::integral_constant<Epi, Epi::ADD>{}, F32_{});   // bf16 outputs take the ADD_PRE instance
  } else {
    if (f32out)
      epilogue(std::integral_constant<Epi, Epi::STORE>{}, F32_{});
    else
      epilogue(std::integral_constant<Epi, Epi::STORE>{}, BF16_{});
  }
}

static int tiled_blocks(StreamGemm& g) {
  int b0 = 0;
  for (int i = 0; i < g.nseg; ++i) {
    const int per = g.seg[i].epi == Epi::SITU ? TILE_N / 2 : TILE_N;
    g.seg[i].blocks = (g.seg[i].n_out + per - 1) / per;
    g.seg[i].block0 = b0;
    b0 += g.seg[i].blocks;
  }
  return b0;
}

// Dense calls whose tiles do not fill the CUs split K so that tiles x slices reach about
// one workgroup per CU, each slice keeping at least 16 K steps (512 elements).
int tiled_splitk(const StreamGemm& g0) {
  if (g0.row_to_pair) return 1;
  StreamGemm g = g0;
  const int G = ((g.M + TILE_M - 1) / TILE_M) * tiled_blocks(g);
  int k = 256 / (G > 0 ? G : 1);
  k = min(k, ((g.Kd + (tiled_dual_ok(g) ? g.Kd1 : 0)) / 32) / 16);
  k = min(k, 8);
  return k < 2 ? 1 : k;
}

// Dense launches of whole rounds: with one workgroup per CU, M x n_out outputs in tiles
// that make a whole number of rounds of the 256 CUs plus part of one leave CUs idle in
// that last round. Returns the output columns (a multiple of TILE_N) whose tiles make
// whole rounds, when the tiles of the remaining columns are at most half a round, so that
// a second launch runs them with split K over every CU; n_out when no such split exists.
int tiled_round_cols(int M, int n_out) {
  const long mt = (M + TILE_M - 1) / TILE_M, nb = (n_out + TILE_N - 1) / TILE_N, G = mt * nb;
  if (G <= 256 || G % 256 == 0) return n_out;
  for (long nb1 = nb - 1; nb1 > 0; --nb1)
    if ((mt * nb1) % 256 == 0) return mt * (nb - nb1) <= 128 ? (int)(nb1 * TILE_N) : n_out;
  return n_out;
}

size_t tiled_splitk_bytes(const StreamGemm& g, int ksplit) {
  if (ksplit <= 1) return 0;
  size_t cols = 0;
  for (int i = 0; i < g.nseg; ++i) cols += (size_t)g.seg[i].n_total;
  return (size_t)ksplit * (size_t)g.M * cols * sizeof(float);
}

// Sum of the K slices (in slice order) and the segment's epilogue; one thread per 4
// output columns of one row.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const StreamGemm g, int ptot) {
  const int si = blockIdx.z, row = blockIdx.y;
  const Seg sg = g.seg[si];
  const int col = 4 * (int)(blockIdx.x * 256 + threadIdx.x);
  if (col >= sg.n_out) return;
  int pbase = 0;
  for (int i = 0; i < si; ++i) pbase += g.seg[i].n_total;
  const size_t slice = (size_t)g.M * ptot;
  const float* src = g.part + (size_t)row * ptot + pbase + col;
  floatx4 v = *reinterpret_cast<const floatx4*>(src);
  for (int k = 1; k < g.ksplit; ++k) v += *reinterpret_cast<const floatx4*>(src + k * slice);
  if (sg.epi == Epi::SITU) {
    floatx4 u = *reinterpret_cast<const floatx4*>(src + sg.n_out);
    for (int k = 1; k < g.ksplit; ++k) u += *reinterpret_cast<const floatx4*>(src + sg.n_out + k * slice);
    const float inv_b = 1.0f / g.beta;
    const float inv_lb = g.lbeta > 0.0f ? 1.0f / g.lbeta : 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = situ_f(v[q], u[q], g.beta, inv_b, g.lbeta, inv_lb);
  }
  const size_t idx = (size_t)row * sg.ldo + col;
  if (sg.epi == Epi::ADD && g.add != nullptr) {
    if (sg.out_elt == Elt::F32) {
      v += *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(g.add) + idx);
    } else {
      const uint2 a = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(g.add) + idx);
      v += floatx4{bf16_to_f32((uint16_t)a.x), bf16_to_f32((uint16_t)(a.x >> 16)), bf16_to_f32((uint16_t)a.y),
                   bf16_to_f32((uint16_t)(a.y >> 16))};
    }
  }
  if (sg.out_elt == Elt::F32) {
    *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(sg.out) + idx) = v;
  } else {
    const uint32_t lo = pack_bf16x2(v[0], v[1]);
    const uint32_t hi = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(sg.out) + idx) = make_uint2(lo, hi);
  }
}

// Two K phases in one launch (sums of both products in one set of fp32 accumulators):
// dense, one plain-store segment, a second phase (Kd1 > 0: a1 and w1 are its operands).
bool tiled_dual_ok(const StreamGemm& g) {
  return g.Kd1 > 0 && g.row_to_pair == nullptr && g.nseg == 1 && g.seg[0].epi == Epi::STORE && g.Kd % 32 == 0 &&
         g.Kd1 % 32 == 0;
}

hipError_t launch_tiled_gemm(StreamGemm g, hipStream_t stream) {
  // two K phases: dense, one plain-store segment (see the kernel); split-K slices cut the
  // steps of both phases together
  const bool dual = tiled_dual_ok(g);
  const int nch = g.Kd / 32 + (dual ? g.Kd1 / 32 : 0);
  const int b0 = tiled_blocks(g);
  if (g.ksplit < 2 || !g.part || g.row_to_pair) g.ksplit = 1;
  const int m_tiles = (g.M + TILE_M - 1) / TILE_M;
  // a multiple of 8 workgroups (dense) or whole rounds of 8 groups (grouped); the ids past
  // the tiles return at once
  const long n = (long)m_tiles * b0 * g.ksplit;
  const long per_group = (long)GROUP_M * b0;
  const unsigned grid = g.row_to_pair ? (unsigned)(((n + per_group - 1) / per_group + 7) / 8 * 8 * per_group)
                                      : (unsigned)((n + 7) & ~7L);
  const bool add_pre = g.nseg == 1 && g.seg[0].epi == Epi::ADD && g.add != nullptr && g.seg[0].out_elt == Elt::BF16 &&
                       g.ksplit == 1;
  if (dual)
    hipLaunchKernelGGL((tiled_gemm_kernel<false, true>), dim3(grid), dim3(512), 0, stream, g, b0, m_tiles, nch);
  else if (add_pre)
    hipLaunchKernelGGL((tiled_gemm_kernel<true, false>), dim3(grid), dim3(512), 0, stream, g, b0, m_tiles, nch);
  else
    hipLaunchKernelGGL((tiled_gemm_kernel<false, false>), dim3(grid), dim3(512), 0, stream, g, b0, m_tiles, nch);
  if (g.ksplit > 1) {
    int ptot = 0, wmax = 0;
    for (int i = 0; i < g.nseg; ++i) {
      ptot += g.seg[i].n_total;
      wmax = max(wmax, g.seg[i].n_out);
    }
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((wmax / 4 + 255) / 256), (unsigned)g.M, (unsigned)g.nseg),
                       dim3(256), 0, stream, g, ptot);
  }
  return hipGetLastError();
}

}  // namespace lmoe
