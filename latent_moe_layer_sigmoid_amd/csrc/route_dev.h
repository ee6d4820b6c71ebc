// Device routine of single-group sigmoid top-k routing for gfx950, shared by the routing
// kernel and the fused routing + permutation kernel. The method and the data layout are
// described in route.hip.
#pragma once
#include "common.h"

namespace lmoe {

LMOE_DEV uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Maximum of x over the 64 lanes, returned as a wave-uniform value.
// Row shifts 1, 2, 4, 8 leave each row's maximum in its lane 15; two row broadcasts
// carry it to lane 63. Lanes reading outside their row see 0, the identity here.
LMOE_DEV uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true));   // row_shr:1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true));   // row_shr:2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true));   // row_shr:4
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true));   // row_shr:8
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Sort keys are positive normal doubles: the bits 2^52 + s 2^10 + (1023 - e) for the
// order-preserving 32 bits s of an expert's fp32 key and its index e < 1024, so that the
// fp64 order is that of s, then of the lower index; padding is 2^52 itself (s = 0, which
// no real key has), below every real key. A compare-exchange is then one fp64 max and one
// fp64 min (each returns one of its operands unchanged), with no condition register
// between the comparators, which a 64-bit integer compare and four selects would need.
LMOE_DEV double sort_key(uint32_t s, int e) {
  return __builtin_bit_cast(double, (1ull << 52) | ((uint64_t)s << 10) | (uint64_t)(1023 - e));
}
constexpr double kSortPad = 2.2250738585072014e-308;   // the double with bits 2^52
LMOE_DEV uint32_t sort_key_s(double k) { return (uint32_t)((__builtin_bit_cast(uint64_t, k) >> 10) & 0xFFFFFFFFull); }
LMOE_DEV int sort_key_e(double k) { return 1023 - (int)(__builtin_bit_cast(uint64_t, k) & 1023ull); }

LMOE_DEV void cas_desc(double& a, double& b) {
  const double hi = __builtin_fmax(a, b), lo = __builtin_fmin(a, b);
  a = hi;
  b = lo;
}

// Batcher's odd-even merge sort of N (a power of two) keys, descending; fully unrolled.
// Keys from index LIVE on are padding, below every real key: a descending
// compare-exchange leaves the smaller key at the higher index, so such a slot only ever
// meets real keys as the higher index and keeps its padding; those comparators are left out.
template <int N, int LIVE = N>
LMOE_DEV void sort_desc(double* k) {
#pragma unroll
  for (int p = 1; p < N; p <<= 1)
#pragma unroll
    for (int q = p; q >= 1; q >>= 1)
#pragma unroll
      for (int j = q % p; j + q < N; j += 2 * q)
#pragma unroll
        for (int i = 0; i < q; ++i)
          if (i + j + q < LIVE && (i + j) / (2 * p) == (i + j + q) / (2 * p)) cas_desc(k[i + j], k[i + j + q]);
}

LMOE_DEV float score_of(float logit) { return __builtin_amdgcn_rcpf(1.0f + __expf(-logit)); }

// Selection key of one expert: METHOD 0 (sigmoid scores with the selection bias, [P1]
// commit 4) gives sigmoid(logit) + bias; METHOD 1 ("Renormalize": logits cast to bf16,
// no bias) gives the bf16 value of the logit.
template <int METHOD>
LMOE_DEV float route_key(float logit, float bias) {
  if (METHOD == 0) return score_of(logit) + bias;
  return bf16_to_f32(f32_to_bf16(logit));
}

// Routes token t with the calling wavefront: lane k < K returns expert *e and weight *w of
// slot k (other lanes return e = -1). Every lane of the wavefront must call it.
// group_size > 0: only experts whose group (e / group_size) has its bit set in the
// wave-uniform keep_groups mask compete (grouped top-k).
// Weights: METHOD 0 -- rsf * s / sum(s) over the K winners' unbiased scores (or rsf * s
// without renorm); METHOD 1 -- softmax of the K winners' bf16 logits.
//
// Each lane keeps its sorted keys in a register vector and a head index; a round reads
// registers at wave-uniform indices only (the winning lane's next key, the winner's logit
// slot), which compile to relative register moves rather than per-slot selects. The
// second (expert index) reduction runs only when several lanes hold the top score.
template <int KPL, int NP, int METHOD = 0>
LMOE_DEV void route_token(int t, int E, int K, const float* __restrict__ logits, const float* __restrict__ bias,
                          float rsf, int renorm, int* e_out, float* w_out, int group_size = 0,
                          uint64_t keep_groups = ~0ull) {
  typedef uint32_t u32v __attribute__((ext_vector_type(NP)));
  typedef float f32v __attribute__((ext_vector_type(NP)));
  const int lane = threadIdx.x & 63;
  const float* row = logits + (size_t)t * E;

  // issue every load before the first use (clamped, in-bounds indices), then build keys
  float lg[KPL], bs[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int e = min(lane + 64 * j, E - 1);
    lg[j] = row[e];
    bs[j] = (METHOD == 0 && bias) ? bias[e] : 0.0f;
  }
  double key[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int e = lane + 64 * j;
    key[j] = kSortPad;   // below every real key; never selected since K <= the competing experts
    const bool competes = e < E && (group_size <= 0 || ((keep_groups >> (e / max(group_size, 1))) & 1ull));
    if (j < KPL && competes) key[j] = sort_key(orderable(route_key<METHOD>(lg[j], bs[j])), e);
  }
  sort_desc<NP, KPL>(key);
  // the selection rounds work on two 32-bit words per key: the score bits (0 for padding)
  // and ~expert
  u32v vh, vl;
  f32v vlg;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    vh[j] = sort_key_s(key[j]);
    vl[j] = 0xFFFFFFFFu - (uint32_t)sort_key_e(key[j]);
    vlg[j] = j < KPL ? lg[j] : 0.0f;
  }

  uint32_t hh = vh[0], ll = vl[0];   // this lane's current head key
  int head = 0;
  uint32_t my_lo = 0;
  float my_lg = 0.0f;
  auto round = [&](int k) __attribute__((always_inline)) {
    const uint32_t mh = wave_max_u32(hh);
    const uint64_t tied = __ballot(hh == mh);
    int wl;
    uint32_t ml;
    if (__builtin_expect(__popcll(tied) == 1, 1)) {   // ties are rare: the other path out of line
      wl = __ffsll((unsigned long long)tied) - 1;
      ml = (uint32_t)__builtin_amdgcn_readlane((int)ll, wl);
    } else {   // equal scores: the larger ~expert (lower expert index) wins
      ml = wave_max_u32(hh == mh ? ll : 0u);
      wl = __ffsll((unsigned long long)__ballot(hh == mh && ll == ml)) - 1;
    }
    // the winner's logit: register slot e / 64 of lane e % 64 (both wave-uniform). The slot
    // index goes through readfirstlane: written directly inside the readlane operand, the
    // compiler has been seen to drop the vector index (always reading slot 0).
    const uint32_t ew = 0xFFFFFFFFu - ml;
    const int jw = __builtin_amdgcn_readfirstlane((int)(ew >> 6) & (NP - 1));
    const float xw = vlg[jw];
    const float lw = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, xw), (int)(ew & 63)));
    if (lane == k) {
      my_lo = ml;
      my_lg = lw;
    }
    // the winning lane moves its head to its next key
    const int nxt = __builtin_amdgcn_readlane(head, wl) + 1;
    const uint32_t nh = nxt < NP ? vh[nxt & (NP - 1)] : 0u;
    const uint32_t nl = nxt < NP ? vl[nxt & (NP - 1)] : 0u;
    if (lane == wl) {
      hh = nh;
      ll = nl;
      head = nxt;
    }
  };
  // top-16 and top-8, the common cases, as straight code: no loop branch between rounds,
  // and one round's tail overlaps the next one's maximum (measured at top-16: 5.9 -> 5.2 us
  // per call of 1024 tokens)
  if (K == 16) {
    static_for<16>([&](auto k) __attribute__((always_inline)) { round(decltype(k)::value); });
  } else if (K == 8) {
    static_for<8>([&](auto k) __attribute__((always_inline)) { round(decltype(k)::value); });
  } else {
    for (int k = 0; k < K; ++k) round(k);
  }
  int e = -1;
  float s = 0.0f;
  if (METHOD == 0) {
    if (lane < K) {
      e = (int)(0xFFFFFFFFu - my_lo);
      s = score_of(my_lg);   // same expression as at selection time
    }
  } else {
    // softmax over the winners: slot 0 holds the largest bf16 logit
    const float v = route_key<1>(my_lg, 0.0f);
    const float vmax = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    if (lane < K) {
      e = (int)(0xFFFFFFFFu - my_lo);
      s = __expf(v - vmax);
    }
  }
  float sum = s;            // butterfly: every lane ends with the same total
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) sum += __shfl_xor(sum, off, WAVE);
  *e_out = e;
  if (METHOD == 0)
    *w_out = renorm ? rsf * s / sum : rsf * s;
  else
    *w_out = s / sum;
}

}  // namespace lmoe
