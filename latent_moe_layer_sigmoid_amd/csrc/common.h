// Device helpers shared by the gfx950 kernels of the latent-MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#define LMOE_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));

namespace lmoe {

constexpr int WAVE = 64;

LMOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bfloat16, round to nearest even (NaN stays NaN): the gfx950 conversion
// instruction (v_cvt_pk_bf16_f32), which rounds in the default nearest-even mode.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
LMOE_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two floats -> two bfloat16 in one 32-bit word (lo in the low half), one instruction
LMOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){lo, hi}, bf16x2_t));
}

// Hardware transcendental building blocks (v_exp_f32 / v_rcp_f32).
LMOE_DEV float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
LMOE_DEV float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
LMOE_DEV float fast_sigmoid(float x) { return fast_rcp(1.0f + fast_exp(-x)); }
// tanh(x). For |x| >= 0.3: 1 - 2 / (exp(2x) + 1), which saturates cleanly to +-1 when
// exp overflows or underflows. Below 0.3 that form loses relative accuracy as |x| -> 0
// (1 minus a quotient near 1), so the odd Taylor series is used there up to x^9: the
// first omitted term, 1382 x^11 / 155925, is below 6e-8 of tanh(x) at |x| = 0.3.
LMOE_DEV float fast_tanh(float x) {
  const float big = 1.0f - 2.0f * fast_rcp(fast_exp(2.0f * x) + 1.0f);
  const float x2 = x * x;
  float p = 62.0f / 2835.0f;
  p = __builtin_fmaf(p, x2, -17.0f / 315.0f);
  p = __builtin_fmaf(p, x2, 2.0f / 15.0f);
  p = __builtin_fmaf(p, x2, -1.0f / 3.0f);
  const float small = __builtin_fmaf(p * x2, x, x);
  return __builtin_fabsf(x) < 0.3f ? small : big;
}

// exp(x) - 1: the Taylor series to x^7 for |x| < 0.3 (first omitted term below 2e-9 of
// the result), e^x - 1 otherwise.
LMOE_DEV float fast_expm1(float x, float ex) {
  float p = 1.0f + x * (1.0f / 7.0f);
  p = 1.0f + x * (1.0f / 6.0f) * p;
  p = 1.0f + x * (1.0f / 5.0f) * p;
  p = 1.0f + x * (1.0f / 4.0f) * p;
  p = 1.0f + x * (1.0f / 3.0f) * p;
  p = 1.0f + x * 0.5f * p;
  return __builtin_fabsf(x) < 0.3f ? x * p : ex - 1.0f;
}

// SituGLU of one (gate, up) pair in fp32: beta*tanh(g/beta)*sigmoid(g) times
// (linear_beta > 0 ? linear_beta*tanh(u/linear_beta) : u).
// With beta = 1 the gate needs one exponential: with E = e^g,
// tanh(g) * sigmoid(g) = (E^2 - 1) / (E^2 + 1) * E / (E + 1) = E (E - 1) / (E^2 + 1),
// where E - 1 comes from fast_expm1 (accurate near g = 0); g is clamped to [-87, 40]
// (beyond it the product is 1 to fp32 precision above and e^g to fp32 range below).
LMOE_DEV float situ_f(float g, float u, float beta, float inv_beta, float lbeta, float inv_lbeta) {
  float gate;
  if (beta == 1.0f) {
    const float gc = __builtin_fminf(__builtin_fmaxf(g, -87.0f), 40.0f);
    const float ex = fast_exp(gc);
    const float em1 = fast_expm1(gc, ex);
    gate = em1 * ex * fast_rcp(__builtin_fmaf(ex, ex, 1.0f));
  } else {
    gate = beta * fast_tanh(g * inv_beta) * fast_sigmoid(g);
  }
  const float up = lbeta > 0.0f ? lbeta * fast_tanh(u * inv_lbeta) : u;
  return gate * up;
}

// FP8 E4M3 ("fn") code of v: round to nearest even, saturate at +-448; sign bit for v < 0.
LMOE_DEV uint32_t e4m3_encode(float v) {
  uint32_t sign = v < 0.0f ? 0x80u : 0u;
  float a = fabsf(v);
  if (!(a < 464.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid of 2^-9
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  int E = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;   // floor(log2 a), a normal
  float q = __builtin_rintf(__builtin_ldexpf(a, 3 - E));   // in [8, 16]
  return sign | (uint32_t)(((E + 7) << 3) + (int)q - 8);
}

LMOE_DEV float e4m3_decode(uint32_t c) {
  uint32_t e = (c >> 3) & 0xF, m = c & 7;
  float mag = e == 0 ? (float)m * 0.001953125f : __builtin_ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
  return (c & 0x80) ? -mag : mag;
}

// Shared MX exponent of a block whose absolute maximum is amax:
// floor(log2 amax) - 8, clamped to [-127, 127]; 0 for an all-zero block.
LMOE_DEV int mx_e4m3_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e;
  (void)__builtin_frexpf(amax, &e);          // amax = m * 2^e, m in [0.5, 1)
  int x = e - 1 - 8;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// Buffer resource: wave-uniform base address and byte size; the hardware range-checks
// every access (reads past the end return zeros, writes past it are dropped).
typedef __amdgpu_buffer_rsrc_t rsrc_t;

LMOE_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// ---- buffer-to-LDS copies and the waits around them (tiled and MX GEMMs)
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediates (gfx9 encoding): vm = vector-memory count (6 bits), lgkm = LDS
// count (4 bits); expcnt unconstrained.
constexpr int waitcnt(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8); }

// One wave-wide copy of 16 bytes per lane from a buffer into LDS at lds + 16 * lane.
LMOE_DEV void to_lds(rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// A wave-uniform copy of a pointer / value (kept in scalar registers, so that buffer
// descriptors built from it need no per-lane waterfall).
LMOE_DEV const char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// Workgroup barrier without the release/acquire fences of __syncthreads(): the fence would
// make every wavefront wait for all of its buffer-to-LDS loads, including the ones meant
// to stay in flight. A kernel using it orders LDS itself: s_waitcnt on its own loads, then
// this.
LMOE_DEV void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <typename T>
LMOE_DEV T wave_max(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    T o = __shfl_xor(v, off, WAVE);
    v = o > v ? o : v;
  }
  return v;
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1, so that register
// arrays indexed by I stay in registers.
template <typename F, int... I>
LMOE_DEV void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
LMOE_DEV void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Workgroup barrier that orders LDS accesses only: global stores issued before it are not
// waited for (use it where threads exchange data through LDS alone).
LMOE_DEV void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

LMOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return v;
}

}  // namespace lmoe
