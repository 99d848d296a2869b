// AdamW update of the float32 master weights (nanochat "AdamW Fused Step":
// decay first, then the lerp of the first moment, bias correction, and
// p -= step_size * m / denom; the second moment and denom, which that listing
// leaves out, follow the textbook Adam form sqrt(v) / sqrt(1 - beta2^t) + eps).
//
// This file is compiled with -ffp-contract=off: every multiply and add below
// rounds on its own, division and square root are correctly rounded and
// denormals are kept, so the update is bit-identical to the same sequence of
// IEEE float operations done anywhere else.  One thread handles four
// consecutive elements with 16-byte loads; the bf16 copy of p that the matrix
// products read is written in the same pass.

#include "common.h"
#include "kernels.h"

namespace gpt {

namespace {

// Correctly rounded float square root.  The hardware v_sqrt_f32 is only
// faithful (1 ulp); the double-precision square root is accurate to well under
// 2^-53 relative, and rounding it to float is then exact-to-nearest, because a
// float's square root never lies within 2^-50 (relative) of a float midpoint
// (53 >= 2*24 + 2 bits).
__device__ __forceinline__ float sqrt_rn(float x) { return (float)__dsqrt_rn((double)x); }

__device__ __forceinline__ void adam_one(float& p, float& m, float& v, float g,
                                         const AdamScalars& s) {
  g = g * s.scale;
  p = p * s.decay;
  m = m + s.omb1 * (g - m);
  v = v + s.omb2 * (g * g - v);
  float d = __fdiv_rn(sqrt_rn(v), s.sbc2) + s.eps;
  p = p - s.step_size * __fdiv_rn(m, d);
}

// Each thread takes two float4 groups per sweep (all eight loads in flight
// before any arithmetic); the arrays are streamed once, so the stores are
// marked non-temporal.
__device__ __forceinline__ void adam4(float4& pp, float4& mm, float4& vv, const float4& gg,
                                      const AdamScalars& s) {
  adam_one(pp.x, mm.x, vv.x, gg.x, s);
  adam_one(pp.y, mm.y, vv.y, gg.y, s);
  adam_one(pp.z, mm.z, vv.z, gg.z, s);
  adam_one(pp.w, mm.w, vv.w, gg.w, s);
}
__device__ __forceinline__ void store4_nt(float* q, const float4& v) {
  __builtin_nontemporal_store(v.x, q);
  __builtin_nontemporal_store(v.y, q + 1);
  __builtin_nontemporal_store(v.z, q + 2);
  __builtin_nontemporal_store(v.w, q + 3);
}

__global__ void __launch_bounds__(256) adamw_kernel(int64_t n, float* __restrict__ p,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    const float* __restrict__ g,
                                                    bf16_t* __restrict__ shadow, AdamScalars s,
                                                    const float* __restrict__ d_scale,
                                                    Guard guard) {
  if (guard_tripped(guard)) return;
  if (d_scale) {  // gradient scale from the device clip; NaN: non-finite norm, no update
    const float sc = *d_scale;
    if (sc != sc) return;
    s.scale = sc;
  }
  const int64_t half = (int64_t)gridDim.x * 256 * 4;  // elements covered by one float4 per thread
  const int64_t stride = 2 * half;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += stride) {
    const int64_t i2 = i + half;
    if (i2 + 3 < n) {
      float4 p0 = *(float4*)(p + i), m0 = *(float4*)(m + i), v0 = *(float4*)(v + i);
      float4 g0 = *(const float4*)(g + i);
      float4 p1 = *(float4*)(p + i2), m1 = *(float4*)(m + i2), v1 = *(float4*)(v + i2);
      float4 g1 = *(const float4*)(g + i2);
      adam4(p0, m0, v0, g0, s);
      adam4(p1, m1, v1, g1, s);
      store4_nt(p + i, p0);
      store4_nt(m + i, m0);
      store4_nt(v + i, v0);
      store4_nt(p + i2, p1);
      store4_nt(m + i2, m1);
      store4_nt(v + i2, v1);
      if (shadow) {
        *(uint2*)(shadow + i) = make_uint2(pack_bf2(p0.x, p0.y), pack_bf2(p0.z, p0.w));
        *(uint2*)(shadow + i2) = make_uint2(pack_bf2(p1.x, p1.y), pack_bf2(p1.z, p1.w));
      }
    } else {
      for (int64_t base : {i, i2}) {
        for (int64_t j = base; j < min(n, base + 4); ++j) {
          float pj = p[j], mj = m[j], vj = v[j];
          adam_one(pj, mj, vj, g[j], s);
          p[j] = pj;
          m[j] = mj;
          v[j] = vj;
          if (shadow) shadow[j] = f2bf(pj);
        }
      }
    }
  }
}

// AdamW over a list of segments of the flat vectors in one launch.  seg holds
// (begin, length, first block) per segment, lengths multiples of 4, each
// segment covered by consecutive blocks of ADAM_SEG_CHUNK elements.
constexpr int ADAM_SEG_CHUNK = 256 * 8;

__global__ void __launch_bounds__(256) adamw_segments_kernel(
    const int64_t* __restrict__ seg, int nseg, float* __restrict__ p, float* __restrict__ m,
    float* __restrict__ v, const float* __restrict__ g, bf16_t* __restrict__ shadow,
    AdamScalars s, Guard guard) {
  if (guard_tripped(guard)) return;
  int lo = 0, hi = nseg - 1;  // the last segment whose first block <= this block
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg[3 * mid + 2] <= (int64_t)blockIdx.x) lo = mid; else hi = mid - 1;
  }
  const int64_t b = seg[3 * lo], end = b + seg[3 * lo + 1];
  const int64_t base = b + ((int64_t)blockIdx.x - seg[3 * lo + 2]) * ADAM_SEG_CHUNK;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t i = base + h * (ADAM_SEG_CHUNK / 2) + threadIdx.x * 4;
    if (i + 3 < end) {
      float4 p0 = *(float4*)(p + i), m0 = *(float4*)(m + i), v0 = *(float4*)(v + i);
      const float4 g0 = *(const float4*)(g + i);
      adam4(p0, m0, v0, g0, s);
      store4_nt(p + i, p0);
      store4_nt(m + i, m0);
      store4_nt(v + i, v0);
      if (shadow) *(uint2*)(shadow + i) = make_uint2(pack_bf2(p0.x, p0.y), pack_bf2(p0.z, p0.w));
    }
  }
}

// The global-norm clip of a step on the device, in the host rule's double
// arithmetic: norm = sqrt(sum g^2) / n_micro, c = max_norm / norm if
// max_norm > 0 and norm > max_norm (else 1), grad_scale = c / n_micro.
// out = {norm, grad_scale}; scale = (float) grad_scale, NaN if the norm is not
// finite or the guard is tripped.
__global__ void clip_scale_kernel(const double* __restrict__ norm2, int n_micro, double max_norm,
                                  double* __restrict__ out, float* __restrict__ scale,
                                  Guard guard) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  const double norm = sqrt(*norm2) / (double)n_micro;
  const double c = (max_norm > 0.0 && norm > max_norm) ? max_norm / norm : 1.0;
  const double sc = c / (double)n_micro;
  const bool finite = norm - norm == 0.0 && !guard_tripped(guard);
  out[0] = norm;
  out[1] = finite ? sc : __builtin_nan("");
  *scale = finite ? (float)sc : __builtin_nanf("");
}

}  // namespace

hipError_t clip_scale(const double* norm2, int n_micro, double max_norm, double* out, float* scale,
                      Guard guard, hipStream_t s) {
  clip_scale_kernel<<<1, 64, 0, s>>>(norm2, n_micro, max_norm, out, scale, guard);
  return hipGetLastError();
}

int adamw_segment_blocks(int64_t len) { return (int)cdiv(len, ADAM_SEG_CHUNK); }

hipError_t adamw_segments(const int64_t* d_seg, int nseg, int blocks, float* p, float* m,
                          float* v, const float* g, uint16_t* shadow, AdamScalars sc,
                          Guard guard, hipStream_t s) {
  if (nseg <= 0 || blocks <= 0) return hipSuccess;
  adamw_segments_kernel<<<(unsigned)blocks, 256, 0, s>>>(d_seg, nseg, p, m, v, g, shadow, sc,
                                                         guard);
  return hipGetLastError();
}

hipError_t adamw(int64_t n, float* p, float* m, float* v, const float* g, uint16_t* shadow,
                 AdamScalars sc, hipStream_t s, const float* d_scale, Guard guard) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = cdiv(cdiv(n, 8), 256);
  if (blocks > 8192) blocks = 8192;
  adamw_kernel<<<(unsigned)blocks, 256, 0, s>>>(n, p, m, v, g, shadow, sc, d_scale, guard);
  return hipGetLastError();
}

}  // namespace gpt
