// Shared device helpers for the gfx950 kernels: bf16 storage, vector
// types, wavefront (64-lane) reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 storage (upper half of an fp32)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MTB_DEV __device__ __forceinline__

MTB_DEV float bf2f(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even (gfx950: one v_cvt_pk_bf16_f32)
MTB_DEV bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// two fp32 -> packed bf16 pair (lo in bits 0..15)
MTB_DEV uint32_t pack2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
MTB_DEV float lo_f(uint32_t p) { return __uint_as_float(p << 16); }
MTB_DEV float hi_f(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// element access by dtype
template <typename T> MTB_DEV float ld_f(const T* p);
template <> MTB_DEV float ld_f<float>(const float* p) { return *p; }
template <> MTB_DEV float ld_f<bf16_t>(const bf16_t* p) { return bf2f(*p); }
template <typename T> MTB_DEV void st_f(T* p, float v);
template <> MTB_DEV void st_f<float>(float* p, float v) { *p = v; }
template <> MTB_DEV void st_f<bf16_t>(bf16_t* p, float v) { *p = f2bf(v); }

// 8 consecutive elements <-> 8 floats
template <typename T> MTB_DEV void ld8(const T* p, float (&v)[8]);
template <> MTB_DEV void ld8<bf16_t>(const bf16_t* p, float (&v)[8]) {
  u32x4 q = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = lo_f(q[i]); v[2 * i + 1] = hi_f(q[i]); }
}
template <> MTB_DEV void ld8<float>(const float* p, float (&v)[8]) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}
template <typename T> MTB_DEV void st8(T* p, const float (&v)[8]);
template <> MTB_DEV void st8<bf16_t>(bf16_t* p, const float (&v)[8]) {
  u32x4 q;
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = pack2(v[2 * i], v[2 * i + 1]);
  *reinterpret_cast<u32x4*>(p) = q;
}
template <> MTB_DEV void st8<float>(float* p, const float (&v)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

// 4 consecutive elements <-> 4 floats
template <typename T> MTB_DEV void ld4(const T* p, float (&v)[4]);
template <> MTB_DEV void ld4<bf16_t>(const bf16_t* p, float (&v)[4]) {
  u32x2 q = *reinterpret_cast<const u32x2*>(p);
  v[0] = lo_f(q[0]); v[1] = hi_f(q[0]); v[2] = lo_f(q[1]); v[3] = hi_f(q[1]);
}
template <> MTB_DEV void ld4<float>(const float* p, float (&v)[4]) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
}
template <typename T> MTB_DEV void st4(T* p, const float (&v)[4]);
template <> MTB_DEV void st4<bf16_t>(bf16_t* p, const float (&v)[4]) {
  u32x2 q;
  q[0] = pack2(v[0], v[1]);
  q[1] = pack2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(p) = q;
}
template <> MTB_DEV void st4<float>(float* p, const float (&v)[4]) {
  f32x4 a = {v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p) = a;
}

// full-wavefront (64 lanes) butterfly reductions
MTB_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
MTB_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// e^x through the hardware base-2 exponential
MTB_DEV float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
MTB_DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// erf(x) from Abramowitz & Stegun, Handbook of Mathematical Functions, eq.
// 7.1.26 (absolute error <= 1.5e-7): for x >= 0, 1 - (a1 t + a2 t^2 + a3 t^3 +
// a4 t^4 + a5 t^5) exp(-x^2) with t = 1 / (1 + p x); odd in x. One branch-free
// path (hardware reciprocal and exp2), so the GEMM epilogues that apply GELU
// to every output element stay cheap. Also returns e = exp(-x^2).
MTB_DEV float erf_as(float x, float& e) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, fabsf(x), 1.0f));
  e = __builtin_amdgcn_exp2f(-x * x * 1.4426950408889634f);
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f),
               0.254829592f);
  return copysignf(1.0f - poly * e, x);
}
// exact-form GELU u * Phi(u), Phi(u) = (1 + erf(u / sqrt 2)) / 2
MTB_DEV float gelu_f(float u) {
  float e;
  return 0.5f * u * (1.0f + erf_as(u * 0.70710678118654752f, e));
}
// GELU'(u) = Phi(u) + u phi(u); phi(u) = exp(-u^2 / 2) / sqrt(2 pi) is the e of erf_as
MTB_DEV float gelu_grad_f(float u) {
  float e;
  const float cdf = 0.5f * (1.0f + erf_as(u * 0.70710678118654752f, e));
  return cdf + u * 0.39894228040143268f * e;
}
// logistic sigmoid 1 / (1 + e^-u) from the hardware base-2 exponential and
// reciprocal (a few instructions instead of the library exp and an IEEE
// division, which made the SwiGLU epilogues VALU-bound); u -> -inf gives
// rcp(inf) = 0, u -> +inf gives 1
MTB_DEV float sigmoid_f(float u) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u * 1.4426950408889634f));
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds; each multiplies counter words 0 and
// 2 by fixed constants and feeds the high halves, xor-ed with the key and the
// other two words, into the next counter; the key advances by two Weyl
// constants between rounds.
MTB_DEV u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                            uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}
