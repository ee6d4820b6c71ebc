// Bandwidth-bound kernels of the layer for gfx950: masked SituGLU, MXFP8 quantization,
// the fixed-order combine of per-pair expert outputs and the latent RMSNorm.
// All use 16-byte (or wider) coalesced accesses; no MFMA (nothing here is a contraction).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace lmoe {

// ---- masked SituGLU over [E, T_max, 2d] (vLLM PR 50088, commit 2: the masked kernel takes
// each expert's valid row count and never touches rows past it; fp32 math).
// The valid rows of all experts (v_e = min(count_e, T_max) each) are one list of
// R = sum v_e rows, dealt evenly to a fixed grid: every workgroup scans the E counts in
// LDS, then wavefront g of the grid takes list rows g, g + G, g + 2G, ... (G wavefronts in
// all), MASK_ROWS rows per trip: it finds each row's expert by a binary search of the
// scanned counts, issues the loads of all of them, then computes and stores. A few
// heavily loaded experts thus do not leave one workgroup with most of the work, and no
// workgroup is launched for rows that do not exist.
constexpr int MASK_ROWS = 4;
constexpr int MASK_MAX_E = 4096;       // experts held in LDS (larger E: one workgroup per expert row chunk)

template <Elt ELT>
struct MaskVec {   // one vector: 8 gate and 8 up values as loaded
  uint4 g[ELT == Elt::BF16 ? 1 : 2], u[ELT == Elt::BF16 ? 1 : 2];
};

template <Elt ELT>
LMOE_DEV void mask_load(const void* in, size_t idx, uint4* v) {
  if (ELT == Elt::BF16) {
    v[0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(in) + idx);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(in) + idx);
    v[0] = p[0];
    v[1] = p[1];
  }
}

template <Elt ELT>
LMOE_DEV void mask_compute_store(const MaskVec<ELT>& q, void* out, size_t oidx, float beta, float inv_b, float lbeta,
                                 float inv_lb) {
  float g[8], u[8];
#pragma unroll
  for (int h = 0; h < (ELT == Elt::BF16 ? 1 : 2); ++h) {
    const uint32_t gw[4] = {q.g[h].x, q.g[h].y, q.g[h].z, q.g[h].w};
    const uint32_t uw[4] = {q.u[h].x, q.u[h].y, q.u[h].z, q.u[h].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ELT == Elt::BF16) {
        g[2 * i] = __uint_as_float(gw[i] << 16);
        g[2 * i + 1] = __uint_as_float(gw[i] & 0xFFFF0000u);
        u[2 * i] = __uint_as_float(uw[i] << 16);
        u[2 * i + 1] = __uint_as_float(uw[i] & 0xFFFF0000u);
      } else {
        g[4 * h + i] = __uint_as_float(gw[i]);
        u[4 * h + i] = __uint_as_float(uw[i]);
      }
    }
  }
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = situ_f(g[i], u[i], beta, inv_b, lbeta, inv_lb);
  if (ELT == Elt::BF16) {
    uint4 ov;
    ov.x = pack_bf16x2(o[0], o[1]);
    ov.y = pack_bf16x2(o[2], o[3]);
    ov.z = pack_bf16x2(o[4], o[5]);
    ov.w = pack_bf16x2(o[6], o[7]);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + oidx) = ov;
  } else {
    float4* op = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + oidx);
    op[0] = make_float4(o[0], o[1], o[2], o[3]);
    op[1] = make_float4(o[4], o[5], o[6], o[7]);
  }
}

template <Elt ELT>
__global__ __launch_bounds__(256) void situ_masked_kernel(int E, int T_max, int d, const void* __restrict__ in,
                                                          const int32_t* __restrict__ counts, float beta,
                                                          float lbeta, void* __restrict__ out) {
  __shared__ int s_off[MASK_MAX_E + 1];   // exclusive prefix of the clamped counts
  __shared__ int s_tot[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // clamped counts and their exclusive scan (chunks of 256 experts, running total); every
  // chunk's counts are requested before the first scan step, so that the loads do not wait
  // on each other across the scan's barriers
  constexpr int NCH = MASK_MAX_E / 256;
  int cv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int e = 256 * i + (int)threadIdx.x;
    cv[i] = e < E ? counts[e] : 0;
  }
  int run = 0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int e0 = 256 * i;
    if (e0 >= E) break;
    const int e = e0 + (int)threadIdx.x;
    int v = cv[i];
    v = v < 0 ? 0 : (v > T_max ? T_max : v);
    int x = v;   // inclusive scan within the wave (shift by 1, 2, ... 32 lanes)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, WAVE);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_tot[w] = x;
    lds_sync();
    int before = run;
    for (int j = 0; j < w; ++j) before += s_tot[j];
    if (e < E) s_off[e] = before + x - v;
    run += s_tot[0] + s_tot[1] + s_tot[2] + s_tot[3];
    lds_sync();
  }
  if (threadIdx.x == 0) s_off[E] = run;
  lds_sync();
  const int R = s_off[E];
  const float inv_b = 1.0f / beta, inv_lb = lbeta > 0.0f ? 1.0f / lbeta : 0.0f;
  const int G = (int)gridDim.x * 4;                      // wavefronts in the grid
  const int vpr = d >> 3;                                // vectors per row
  // expert of list row r: the last e with s_off[e] <= r (wave-uniform search)
  auto expert_of = [&](int r) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  for (int r0 = (int)blockIdx.x * 4 + w; r0 < R; r0 += G * MASK_ROWS) {
    size_t irow[MASK_ROWS], orow[MASK_ROWS];
    bool live[MASK_ROWS];
#pragma unroll
    for (int k = 0; k < MASK_ROWS; ++k) {
      const int r = r0 + k * G;
      live[k] = r < R;
      const int e = live[k] ? expert_of(r) : 0;
      const size_t row = (size_t)e * T_max + (size_t)(r - s_off[e]);
      irow[k] = row * (size_t)(2 * d);
      orow[k] = row * (size_t)d;
    }
    for (int c0 = 0; c0 < vpr; c0 += 64) {
      // every load is issued unconditionally (rows past the list and lanes past the row
      // read the trip's first row and the row's last vector instead), so that no branch
      // separates them and all are in flight together; only the stores are masked
      const int c = c0 + lane;
      const size_t cl = (size_t)min(c, vpr - 1) * 8;
      MaskVec<ELT> q[MASK_ROWS];
#pragma unroll
      for (int k = 0; k < MASK_ROWS; ++k) {
        const size_t ir = live[k] ? irow[k] : irow[0];
        mask_load<ELT>(in, ir + cl, q[k].g);
        mask_load<ELT>(in, ir + d + cl, q[k].u);
      }
#pragma unroll
      for (int k = 0; k < MASK_ROWS; ++k)
        if (live[k] && c < vpr) mask_compute_store<ELT>(q[k], out, orow[k] + (size_t)c * 8, beta, inv_b, lbeta, inv_lb);
    }
  }
}

// E above MASK_MAX_E: one workgroup per (expert, 16-row chunk), 8 outputs per thread.
template <Elt ELT>
__global__ __launch_bounds__(256) void situ_masked_chunk_kernel(int T_max, int d, const void* __restrict__ in,
                                                                const int32_t* __restrict__ counts, float beta,
                                                                float lbeta, void* __restrict__ out) {
  const int e = blockIdx.y;
  int v = counts[e];
  v = v < 0 ? 0 : (v > T_max ? T_max : v);
  const int vpr = d >> 3;
  const float inv_b = 1.0f / beta, inv_lb = lbeta > 0.0f ? 1.0f / lbeta : 0.0f;
  const int r_end = min(v, (int)(blockIdx.x + 1) * 16);
  for (int idx = (int)blockIdx.x * 16 * vpr + (int)threadIdx.x; idx < r_end * vpr; idx += 256) {
    const int r = idx / vpr, c = idx - r * vpr;
    const size_t row = (size_t)e * T_max + r;
    MaskVec<ELT> q;
    mask_load<ELT>(in, row * (size_t)(2 * d) + (size_t)c * 8, q.g);
    mask_load<ELT>(in, row * (size_t)(2 * d) + d + (size_t)c * 8, q.u);
    mask_compute_store<ELT>(q, out, row * (size_t)d + (size_t)c * 8, beta, inv_b, lbeta, inv_lb);
  }
}

hipError_t launch_situ_masked(int E, int T_max, int d, Elt elt, const void* in, const int32_t* counts,
                              float beta, float lbeta, void* out, hipStream_t stream) {
  if (E > MASK_MAX_E) {
    const dim3 grid((unsigned)((T_max + 15) / 16), (unsigned)E);
    if (elt == Elt::BF16)
      hipLaunchKernelGGL(situ_masked_chunk_kernel<Elt::BF16>, grid, dim3(256), 0, stream, T_max, d, in, counts, beta,
                         lbeta, out);
    else
      hipLaunchKernelGGL(situ_masked_chunk_kernel<Elt::F32>, grid, dim3(256), 0, stream, T_max, d, in, counts, beta,
                         lbeta, out);
    return hipGetLastError();
  }
  // enough wavefronts for about MASK_ROWS rows each when every row is valid, at most 1024
  // workgroups (four per CU)
  const long rows = (long)E * T_max;
  const unsigned grid = (unsigned)std::max(1L, std::min(1024L, (rows + 4 * MASK_ROWS - 1) / (4 * MASK_ROWS)));
  if (elt == Elt::BF16)
    hipLaunchKernelGGL(situ_masked_kernel<Elt::BF16>, dim3(grid), dim3(256), 0, stream, E, T_max, d, in, counts, beta,
                       lbeta, out);
  else
    hipLaunchKernelGGL(situ_masked_kernel<Elt::F32>, dim3(grid), dim3(256), 0, stream, E, T_max, d, in, counts, beta,
                       lbeta, out);
  return hipGetLastError();
}

// ---- MXFP8 E4M3 quantization along rows (OCP MX v1.0; TensorRT-LLM PR 20541
// "Description": input quantization before the MXE4M3 x MXE2M1 experts).
// Thread = 8 elements; 4 consecutive lanes = one 32-element block.
template <Elt ELT>
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(long nvec, const void* __restrict__ in,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const bool live = idx < nvec;
  float v[8];
  if (live) {
    if (ELT == Elt::BF16) {
      const uint4 q = reinterpret_cast<const uint4*>(in)[idx];
      const uint16_t* s = reinterpret_cast<const uint16_t*>(&q);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = bf16_to_f32(s[i]);
    } else {
      const float4* p = reinterpret_cast<const float4*>(in) + 2 * idx;
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, WAVE));
  amax = fmaxf(amax, __shfl_xor(amax, 2, WAVE));
  if (!live) return;
  const int X = mx_e4m3_exponent(amax);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= e4m3_encode(__builtin_ldexpf(v[i], -X)) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= e4m3_encode(__builtin_ldexpf(v[4 + i], -X)) << (8 * i);
  reinterpret_cast<uint2*>(codes)[idx] = make_uint2(lo, hi);
  if ((idx & 3) == 0) scales[idx >> 2] = (uint8_t)(X + 127);
}

hipError_t launch_quant_mxfp8(int rows, int cols, Elt elt, const void* in, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  const long nvec = (long)rows * cols / 8;
  const dim3 grid((unsigned)((nvec + 255) / 256)), block(256);
  if (elt == Elt::BF16)
    hipLaunchKernelGGL(quant_mxfp8_kernel<Elt::BF16>, grid, block, 0, stream, nvec, in, codes, scales);
  else
    hipLaunchKernelGGL(quant_mxfp8_kernel<Elt::F32>, grid, block, 0, stream, nvec, in, codes, scales);
  return hipGetLastError();
}

// ---- combine: out[t, :] = sum_{k ascending} ws[t*K + k, :]  (weights already applied).
__global__ __launch_bounds__(256) void combine_kernel(int K, int N, const float* __restrict__ ws, int out_bf16,
                                                      void* __restrict__ out) {
  const int t = blockIdx.y;
  const int c4 = blockIdx.x * 256 + threadIdx.x;   // float4 column index
  if (c4 * 4 >= N) return;
  // streaming loads: every product is read once (see combine_norm_kernel)
  const floatx4* src = reinterpret_cast<const floatx4*>(ws + (size_t)t * K * N) + c4;
  floatx4 sv = __builtin_nontemporal_load(src);
  for (int k0 = 1; k0 < K; k0 += 8) {   // requested 8 at a time, added in k order
    floatx4 u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < K) u[j] = __builtin_nontemporal_load(src + (size_t)(k0 + j) * (N / 4));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < K) sv += u[j];
  }
  const float4 s = make_float4(sv[0], sv[1], sv[2], sv[3]);
  if (out_bf16) {
    uint2 o;
    o.x = pack_bf16x2(s.x, s.y);
    o.y = pack_bf16x2(s.z, s.w);
    reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * N)[c4] = o;
  } else {
    reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (size_t)t * N)[c4] = s;
  }
}

hipError_t launch_combine(int T, int K, int N, const float* ws, Elt out_elt, void* out, hipStream_t stream) {
  const dim3 grid((unsigned)((N / 4 + 255) / 256), (unsigned)T), block(256);
  hipLaunchKernelGGL(combine_kernel, grid, block, 0, stream, K, N, ws, out_elt == Elt::BF16 ? 1 : 0, out);
  return hipGetLastError();
}

// ---- latent RMSNorm (vLLM PR 50088, commit 7: normalize the summed routed output):
// n = z / sqrt(mean(z^2) + eps) * gamma in fp32; one workgroup per token row.
//
// Row layout shared by rmsnorm_kernel and combine_norm_kernel, so that both routes give
// the same bits: a workgroup of norm_threads(T, L) threads owns a row; thread i handles the
// column groups c = VW*i + VW*nthreads*it (it = 0, 1, ...) of VW = norm_vw(T) consecutive
// columns, accumulates their squares with fmas in that order, and the per-thread sums are
// added over the wavefront by butterfly and over the wavefronts in index order. Few rows
// (decode) take two columns per thread, so that a row spreads over up to 1024 threads and
// a thread's loads are few; many rows take four.
constexpr int kNormMaxThreads = 1024;
constexpr int kNormKeep = 4;   // column groups per thread kept in registers by combine_norm_kernel

static int norm_vw(int T) { return T < 64 ? 2 : 4; }
static int norm_threads(int T, int L) {
  const int vw = norm_vw(T);
  const int t = (L / vw + 63) / 64 * 64;
  return t > kNormMaxThreads ? kNormMaxThreads : t;
}

template <int VW>
struct Vec;
template <>
struct Vec<2> {
  typedef float2 T;
  LMOE_DEV static float at(const T& v, int q) { return q == 0 ? v.x : v.y; }
  LMOE_DEV static T zero() { return make_float2(0.f, 0.f); }
  LMOE_DEV static void add(T& a, const T& b) { a.x += b.x; a.y += b.y; }
  // streaming (non-temporal) load: the per-pair products are read once, long after they
  // were written, so keeping them in the caches only evicts lines that are still in use
  LMOE_DEV static T ld_stream(const float* p) {
    typedef float f2v __attribute__((ext_vector_type(2)));
    const f2v t = __builtin_nontemporal_load(reinterpret_cast<const f2v*>(p));
    return make_float2(t[0], t[1]);
  }
};
template <>
struct Vec<4> {
  typedef float4 T;
  LMOE_DEV static float at(const T& v, int q) { return q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w)); }
  LMOE_DEV static T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  LMOE_DEV static void add(T& a, const T& b) { a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w; }
  LMOE_DEV static T ld_stream(const float* p) {
    const floatx4 t = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
  }
};

template <int VW>
LMOE_DEV float sq_acc(float ss, const typename Vec<VW>::T& v) {
#pragma unroll
  for (int q = 0; q < VW; ++q) ss = __builtin_fmaf(Vec<VW>::at(v, q), Vec<VW>::at(v, q), ss);
  return ss;
}

// Sum of v over the workgroup (wavefronts in index order); every thread gets the total.
LMOE_DEV float block_sum(float v, float* s_part) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = v;
  lds_sync();   // the z stores before it need not complete
  float t = s_part[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) t += s_part[w];
  return t;
}

// out[c .. c + VW) = v * r * gamma (gamma applied only when present, as in the oracle).
template <int VW>
LMOE_DEV void store_norm(void* out, int out_bf16, size_t idx, const typename Vec<VW>::T& v, float r,
                         const void* gamma, int gamma_bf16, int c) {
  float o[VW];
#pragma unroll
  for (int q = 0; q < VW; ++q) {
    o[q] = Vec<VW>::at(v, q) * r;
    if (gamma)
      o[q] *= gamma_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(gamma)[c + q])
                         : reinterpret_cast<const float*>(gamma)[c + q];
  }
  if (out_bf16) {
    uint16_t* p = reinterpret_cast<uint16_t*>(out) + idx;
    if (VW == 2) {
      *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(o[0], o[1]);
    } else {
      uint2 w;
      w.x = pack_bf16x2(o[0], o[1]);
      w.y = pack_bf16x2(o[VW - 2], o[VW - 1]);
      *reinterpret_cast<uint2*>(p) = w;
    }
  } else {
    typename Vec<VW>::T w;
    float* wf = reinterpret_cast<float*>(&w);
#pragma unroll
    for (int q = 0; q < VW; ++q) wf[q] = o[q];
    *reinterpret_cast<typename Vec<VW>::T*>(reinterpret_cast<float*>(out) + idx) = w;
  }
}

template <int VW>
__global__ __launch_bounds__(kNormMaxThreads) void rmsnorm_kernel(int L, const float* __restrict__ z,
                                                                  const void* __restrict__ gamma, int gamma_bf16,
                                                                  float eps, int out_bf16, void* __restrict__ out) {
  typedef typename Vec<VW>::T V;
  __shared__ float s_part[kNormMaxThreads / 64];
  const int t = blockIdx.x;
  const int step = VW * blockDim.x;
  const float* row = z + (size_t)t * L;
  float ss = 0.0f;
  for (int c = VW * threadIdx.x; c < L; c += step) ss = sq_acc<VW>(ss, *reinterpret_cast<const V*>(row + c));
  const float tot = block_sum(ss, s_part);
  const float r = 1.0f / sqrtf(tot / (float)L + eps);
  for (int c = VW * threadIdx.x; c < L; c += step)
    store_norm<VW>(out, out_bf16, (size_t)t * L + c, *reinterpret_cast<const V*>(row + c), r, gamma, gamma_bf16, c);
}

// ---- combine + latent RMSNorm in one pass per token: z[t, :] = sum_{k ascending} ws[t*K + k, :]
// (stored fp32, the same additions as combine_kernel), then the RMSNorm of rmsnorm_kernel.
// A thread requests the K products of its columns together (up to 16 at a time), so a
// decode-sized batch pays one memory round trip for the whole combine; z is kept in
// registers for the normalization (re-read, own writes only, past kNormKeep groups).
template <int VW>
__global__ __launch_bounds__(kNormMaxThreads) void combine_norm_kernel(int K, int L, const float* __restrict__ ws,
                                                                       float* __restrict__ z,
                                                                       const void* __restrict__ gamma, int gamma_bf16,
                                                                       float eps, int out_bf16,
                                                                       void* __restrict__ out) {
  typedef typename Vec<VW>::T V;
  __shared__ float s_part[kNormMaxThreads / 64];
  const int t = blockIdx.x;
  const int step = VW * blockDim.x;
  float* zrow = z + (size_t)t * L;
  const float* src = ws + (size_t)t * K * L;
  auto combine = [&](int c) __attribute__((always_inline)) {
    V v = Vec<VW>::ld_stream(src + c);
    for (int k0 = 1; k0 < K; k0 += 16) {
      V u[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (k0 + j < K) u[j] = Vec<VW>::ld_stream(src + (size_t)(k0 + j) * L + c);
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (k0 + j < K) Vec<VW>::add(v, u[j]);
    }
    *reinterpret_cast<V*>(zrow + c) = v;
    return v;
  };
  V keep[kNormKeep];
  float ss = 0.0f;
#pragma unroll
  for (int it = 0; it < kNormKeep; ++it) {
    const int c = VW * threadIdx.x + step * it;
    keep[it] = c < L ? combine(c) : Vec<VW>::zero();
    if (c < L) ss = sq_acc<VW>(ss, keep[it]);
  }
  for (int c = VW * threadIdx.x + step * kNormKeep; c < L; c += step) ss = sq_acc<VW>(ss, combine(c));
  const float tot = block_sum(ss, s_part);
  const float r = 1.0f / sqrtf(tot / (float)L + eps);
#pragma unroll
  for (int it = 0; it < kNormKeep; ++it) {
    const int c = VW * threadIdx.x + step * it;
    if (c < L) store_norm<VW>(out, out_bf16, (size_t)t * L + c, keep[it], r, gamma, gamma_bf16, c);
  }
  for (int c = VW * threadIdx.x + step * kNormKeep; c < L; c += step)
    store_norm<VW>(out, out_bf16, (size_t)t * L + c, *reinterpret_cast<const V*>(zrow + c), r, gamma, gamma_bf16, c);
}

hipError_t launch_combine_norm(int T, int K, int L, const float* ws, float* z, const void* gamma, float eps, Elt elt,
                               void* out, hipStream_t stream) {
  const int vw = norm_vw(T);
  if (L % vw != 0) return hipErrorInvalidValue;
  const int bf = elt == Elt::BF16 ? 1 : 0;
  const dim3 grid(T), block(norm_threads(T, L));
  if (vw == 2)
    hipLaunchKernelGGL(combine_norm_kernel<2>, grid, block, 0, stream, K, L, ws, z, gamma, bf, eps, bf, out);
  else
    hipLaunchKernelGGL(combine_norm_kernel<4>, grid, block, 0, stream, K, L, ws, z, gamma, bf, eps, bf, out);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int T, int L, const float* z, const void* gamma, float eps, Elt elt, void* out,
                          hipStream_t stream) {
  const int vw = norm_vw(T);
  if (L % vw != 0) return hipErrorInvalidValue;
  const int bf = elt == Elt::BF16 ? 1 : 0;
  const dim3 grid(T), block(norm_threads(T, L));
  if (vw == 2)
    hipLaunchKernelGGL(rmsnorm_kernel<2>, grid, block, 0, stream, L, z, gamma, bf, eps, bf, out);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<4>, grid, block, 0, stream, L, z, gamma, bf, eps, bf, out);
  return hipGetLastError();
}

// ---- weight packing for the MFMA operand layout. Per matrix [N, Kd] (row-major source),
// 16-row group n16 and K chunk c (256 bytes of a row: 128 bf16 / 64 fp32) form a 4 KB
// block at (n16 * nch + c) * 4096; inside it, byte q*1024 + g*256 + r*16 + i*esize holds
// W[16*n16 + r][c*KCH + q*(KCH/4) + g*(KCH/16) + i]. Thread = one destination 16 bytes.
__global__ __launch_bounds__(256) void pack_weights_kernel(long pieces, int N, int Kd, int esize,
                                                           const uint4* __restrict__ src, uint4* __restrict__ dst) {
  const long p = (long)blockIdx.x * 256 + threadIdx.x;
  if (p >= pieces) return;
  const int kch = 256 / esize;                 // elements per 256-byte chunk row
  const int nch = Kd / kch;
  const long per_matrix = (long)N * Kd * esize / 16;
  const long b = p / per_matrix, pm = p - b * per_matrix;
  const long blk = pm >> 8;
  const int w = (int)(pm & 255), q = w >> 6, l = w & 63, g = l >> 4, r = l & 15;
  const long n16 = blk / nch, c = blk - n16 * nch;
  const long n = n16 * 16 + r;
  const long k0 = c * kch + q * (kch / 4) + g * (kch / 16);
  dst[p] = src[b * per_matrix + (n * Kd + k0) * esize / 16];
}

hipError_t launch_pack_weights(int batch, int N, int Kd, int esize, const void* src, void* dst, hipStream_t stream) {
  const long pieces = (long)batch * N * Kd * esize / 16;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, pieces, N, Kd,
                     esize, (const uint4*)src, (uint4*)dst);
  return hipGetLastError();
}

// ---- MXFP4 weight packing. Per matrix [N, Kd] (codes [N, Kd/2] bytes, two e2m1 per byte,
// scales [N, Kd/32] e8m0), 16-row group n16 and 512-wide K stage s (nst = Kd / 512):
//   codes: 4 KB block at (n16 * nst + s) * 4096; byte q*1024 + g*256 + r*16 + j holds
//          source byte (s*512 + q*128 + g*32) / 2 + j of row 16*n16 + r (j < 16);
//   scales: 256 B block at (n16 * nst + s) * 256; byte (g*16 + r)*4 + q holds the scale
//          of K block s*16 + q*4 + g of row 16*n16 + r.
// Lane l = 16g + r then reads its MFMA q operand (32 e2m1 values) at q*1024 + 16l and its
// four scales as one dword at 4l.
__global__ __launch_bounds__(256) void pack_mxfp4_codes_kernel(long pieces, int N, int Kd,
                                                               const uint4* __restrict__ src, uint4* __restrict__ dst) {
  const long p = (long)blockIdx.x * 256 + threadIdx.x;
  if (p >= pieces) return;
  const int nst = Kd / 512;
  const long per_matrix = (long)N * Kd / 32;        // 16-byte pieces per matrix
  const long b = p / per_matrix, pm = p - b * per_matrix;
  const long blk = pm >> 8;
  const int w = (int)(pm & 255), q = w >> 6, l = w & 63, g = l >> 4, r = l & 15;
  const long n16 = blk / nst, st = blk - n16 * nst;
  const long row = n16 * 16 + r;
  const long byte0 = (st * 512 + q * 128 + g * 32) / 2;
  dst[p] = src[b * per_matrix + (row * (Kd / 2) + byte0) / 16];
}

__global__ __launch_bounds__(256) void pack_mxfp4_scales_kernel(long n, int N, int Kd, const uint8_t* __restrict__ src,
                                                                uint8_t* __restrict__ dst) {
  const long p = (long)blockIdx.x * 256 + threadIdx.x;
  if (p >= n) return;
  const int nst = Kd / 512;
  const long per_matrix = (long)N * Kd / 32;
  const long b = p / per_matrix, pm = p - b * per_matrix;
  const long blk = pm >> 8;
  const int w = (int)(pm & 255), l = w >> 2, q = w & 3, g = l >> 4, r = l & 15;
  const long n16 = blk / nst, st = blk - n16 * nst;
  const long row = n16 * 16 + r;
  dst[p] = src[b * per_matrix + row * (Kd / 32) + st * 16 + q * 4 + g];
}

hipError_t launch_pack_mxfp4(int batch, int N, int Kd, const void* codes_src, const void* scales_src, void* codes_dst,
                             void* scales_dst, hipStream_t stream) {
  const long pieces = (long)batch * N * Kd / 32;
  hipLaunchKernelGGL(pack_mxfp4_codes_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, pieces, N,
                     Kd, (const uint4*)codes_src, (uint4*)codes_dst);
  const long ns = (long)batch * N * Kd / 32;
  hipLaunchKernelGGL(pack_mxfp4_scales_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream, ns, N, Kd,
                     (const uint8_t*)scales_src, (uint8_t*)scales_dst);
  return hipGetLastError();
}

}  // namespace lmoe
