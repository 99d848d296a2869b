// Internal helpers shared by the HIP kernels of the GPT step (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace gpt {

typedef uint16_t bf16_t;  // storage type of bfloat16 values

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// float -> bf16, round to nearest even (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
// Two floats -> packed bf16 pair, lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Type traits for the activation type (float in fp32 mode, bf16 in bf16 mode).
template <typename T> struct Act;
template <> struct Act<float> {
  __device__ __forceinline__ static float load(const float* p, long i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, long i, float v) { p[i] = v; }
};
template <> struct Act<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, long i) { return bf2f(p[i]); }
  __device__ __forceinline__ static void store(bf16_t* p, long i, float v) { p[i] = f2bf(v); }
};

// GELU.  Exact form: u * Phi(u) with erff; tanh form: the Hendrycks-Gimpel
// approximation 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))).
__device__ __forceinline__ float gelu_f(float u, bool tanh_form) {
  if (tanh_form) {
    const float s = 0.7978845608028654f, k = 0.044715f;
    return 0.5f * u * (1.f + tanhf(s * (u + k * u * u * u)));
  }
  return 0.5f * u * (1.f + erff(u * 0.7071067811865476f));
}
__device__ __forceinline__ float gelu_grad_f(float u, bool tanh_form) {
  if (tanh_form) {
    const float s = 0.7978845608028654f, k = 0.044715f;
    float t = tanhf(s * (u + k * u * u * u));
    return 0.5f * (1.f + t) + 0.5f * u * (1.f - t * t) * s * (1.f + 3.f * k * u * u);
  }
  return 0.5f * (1.f + erff(u * 0.7071067811865476f)) +
         u * 0.3989422804014327f * expf(-0.5f * u * u);
}

// Fast GELU for the bf16 path, whose results are rounded to 8 significant
// bits: absolute error ~1e-7 relative to the forms above.
//  tanh form: 0.5 u (1 + tanh z) = u * sigmoid(2 z), z = sqrt(2/pi) (u + 0.044715 u^3),
//    with the hardware exp2 and reciprocal;
//  exact form: erf by Abramowitz & Stegun, Handbook of Mathematical Functions,
//    formula 7.1.26 (|error| <= 1.5e-7), with erf(-x) = -erf(x).
__device__ __forceinline__ float sigmoid2z(float u, float u2) {
  // sigmoid(2 z) of the tanh form, z = s (u + k u^3), s = sqrt(2 / pi),
  // k = 0.044715: the exp2 argument -2 log2(e) z is one polynomial in u
  // (u2 = u * u, shared with the derivative).
  constexpr float c0 = -2.8853900817779268f * 0.7978845608028654f;
  constexpr float c1 = c0 * 0.044715f;
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(u * fmaf(c1, u2, c0)));
}
// erf(|x|) and exp(-x^2) for the exact form.
__device__ __forceinline__ float erf_as(float x, float& ex2) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  ex2 = __builtin_amdgcn_exp2f(-1.4426950408889634f * ax * ax);
  const float e = 1.f - poly * ex2;
  return copysignf(e, x);
}
__device__ __forceinline__ float gelu_fast(float u, bool tanh_form) {
  if (tanh_form) return u * sigmoid2z(u, u * u);
  float ex2;
  return 0.5f * u * (1.f + erf_as(u * 0.7071067811865476f, ex2));
}
__device__ __forceinline__ float gelu_grad_fast(float u, bool tanh_form) {
  if (tanh_form) {
    // d/du [u sigmoid(2z)] = sg (1 + u (1 - sg) 2 z'(u)),  2 z' = 2 s + 6 s k u^2
    constexpr float s2 = 2.f * 0.7978845608028654f, s6k = 6.f * 0.7978845608028654f * 0.044715f;
    const float u2 = u * u;
    const float sg = sigmoid2z(u, u2);
    return sg * fmaf(u * (1.f - sg), fmaf(s6k, u2, s2), 1.f);
  }
  float ex2;
  const float e = erf_as(u * 0.7071067811865476f, ex2);  // ex2 = exp(-u^2 / 2)
  return fmaf(0.5f, e, 0.5f) + u * 0.3989422804014327f * ex2;
}

// GELU(u) and GELU'(u) together (fast forms, shared intermediate values).
__device__ __forceinline__ void gelu_pair_fast(float u, bool tanh_form, float& g, float& gp) {
  if (tanh_form) {
    constexpr float s2 = 2.f * 0.7978845608028654f, s6k = 6.f * 0.7978845608028654f * 0.044715f;
    const float u2 = u * u;
    const float sg = sigmoid2z(u, u2);
    g = u * sg;
    gp = sg * fmaf(u * (1.f - sg), fmaf(s6k, u2, s2), 1.f);
    return;
  }
  float ex2;
  const float e = erf_as(u * 0.7071067811865476f, ex2);
  g = 0.5f * u * (1.f + e);
  gp = fmaf(0.5f, e, 0.5f) + u * 0.3989422804014327f * ex2;
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double warp_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

inline long cdiv(long a, long b) { return (a + b - 1) / b; }

// Token-id guard.  A forward that meets a token id or target outside
// [0, vocab_size) reads a clamped id (0) instead, so no kernel indexes out of
// bounds, and stores its forward count (gen >= 1) at *flag.  Update kernels
// given a Guard skip their writes when the flag holds a forward count >=
// gen_lo (a forward since the last update saw a bad id).  flag == NULL: off.
struct Guard {
  const int32_t* flag;
  int32_t gen_lo;
};
__device__ __forceinline__ bool guard_tripped(const Guard& g) {
  return g.flag != nullptr && *(volatile const int32_t*)g.flag >= g.gen_lo;
}
// id if 0 <= id < n, else 0 with *flag = gen (flag may be NULL).
__device__ __forceinline__ int checked_id(int id, int n, int32_t* flag, int32_t gen) {
  if ((unsigned)id < (unsigned)n) return id;
  if (flag) *(volatile int32_t*)flag = gen;
  return 0;
}

}  // namespace gpt
