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

// float -> bfloat16, round to nearest even (NaN stays NaN).
LMOE_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Hardware transcendental building blocks (v_exp_f32 / v_rcp_f32).
LMOE_DEV float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
LMOE_DEV float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
LMOE_DEV float fast_sigmoid(float x) { return fast_rcp(1.0f + fast_exp(-x)); }
// tanh(x) = 1 - 2 / (exp(2x) + 1); saturates cleanly to +-1 when exp over/underflows.
LMOE_DEV float fast_tanh(float x) { return 1.0f - 2.0f * fast_rcp(fast_exp(2.0f * x) + 1.0f); }

// SituGLU of one (gate, up) pair in fp32: beta*tanh(g/beta)*sigmoid(g) times
// (linear_beta > 0 ? linear_beta*tanh(u/linear_beta) : u).
LMOE_DEV float situ_f(float g, float u, float beta, float inv_beta, float lbeta, float inv_lbeta) {
  float gate = beta * fast_tanh(g * inv_beta) * fast_sigmoid(g);
  float up = lbeta > 0.0f ? lbeta * fast_tanh(u * inv_lbeta) : u;
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
