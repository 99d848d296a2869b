// Memory-bound kernels of the GPT step: embeddings, LayerNorm, bias-gradient
// column sums, fused softmax cross-entropy, loss mean, sum of squares.
//
// All reductions run in a fixed order (no floating-point atomics), so every
// result is bitwise reproducible run to run: the Panthalia plugin page
// ("Conclusion") requires the same inputs and weights to give the same result,
// and the llm.c FAQ notes that bit-level determinism needs kernel care.

#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace gpt {

namespace {

// ------------------------------------------------------------------ embeddings
// x[m, :] = wte[idx[m], :] + wpe[m % T, :]   (nanoGPT README: learned token and
// position embeddings; "todos" lists other position schemes as future work).
__global__ void __launch_bounds__(256) embed_fwd_kernel(const int32_t* idx, const float* wte,
                                                        const float* wpe, int M, int T, int C,
                                                        float* x) {
  const int C4 = C / 4;
  long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)M * C4) return;
  int m = (int)(i / C4), c = (int)(i % C4);
  int tok = idx[m];
  float4 a = ((const float4*)(wte + (long)tok * C))[c];
  float4 b = ((const float4*)(wpe + (long)(m % T) * C))[c];
  ((float4*)(x + (long)m * C))[c] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

__global__ void fill_i32(int32_t* p, int n, int v) {
  int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void embed_count_kernel(const int32_t* idx, int M, int32_t* counts) {
  int i = blockIdx.x * 256 + threadIdx.x;
  if (i < M) atomicAdd(&counts[idx[i]], 1);  // integer: exact in any order
}

// Exclusive scan of counts[n] -> offsets[n] (one workgroup, fixed order).
__global__ void __launch_bounds__(1024) scan_kernel(const int32_t* counts, int n,
                                                    int32_t* offsets) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int b = t * per, e = min(n, b + per);
  int s = 0;
  for (int i = b; i < e; ++i) s += counts[i];
  part[t] = s;
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int i = 0; i < 1024; ++i) {
      int v = part[i];
      part[i] = acc;
      acc += v;
    }
  }
  __syncthreads();
  int acc = part[t];
  for (int i = b; i < e; ++i) {
    offsets[i] = acc;
    acc += counts[i];
  }
}

// perm[offsets[idx[p]] + rank] = p, rank = #{p' < p : idx[p'] == idx[p]}:
// positions grouped by token, increasing within a token.
__global__ void __launch_bounds__(256) embed_rank_kernel(const int32_t* idx, int M,
                                                         const int32_t* offsets, int32_t* perm) {
  __shared__ int32_t tile[256];
  const int p = blockIdx.x * 256 + threadIdx.x;
  const int mine = p < M ? idx[p] : -1;
  int rank = 0;
  for (int t0 = 0; t0 <= blockIdx.x * 256; t0 += 256) {
    __syncthreads();
    tile[threadIdx.x] = (t0 + (int)threadIdx.x < M) ? idx[t0 + threadIdx.x] : -2;
    __syncthreads();
    int lim = min(256, p - t0);
    for (int k = 0; k < lim; ++k) rank += (tile[k] == mine);
  }
  if (p < M) perm[offsets[mine] + rank] = p;
}

// dwte[v, c] (+)= sum over positions of token v, in position order.
__global__ void __launch_bounds__(256) embed_wte_kernel(const float* dx, int C, const int32_t* counts,
                                                        const int32_t* offsets, const int32_t* perm,
                                                        float* dwte, int accumulate) {
  const int v = blockIdx.x;
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= C) return;
  const int n = counts[v];
  float* out = dwte + (long)v * C + c;
  if (n == 0) {
    if (!accumulate) *out = 0.f;
    return;
  }
  const int o = offsets[v];
  float s = 0.f;
  for (int i = 0; i < n; ++i) s += dx[(long)perm[o + i] * C + c];
  *out = accumulate ? *out + s : s;
}

// dwpe[t, c] (+)= sum_b dx[b*T + t, c]; rows t >= T untouched (accumulate) or zeroed.
__global__ void __launch_bounds__(256) embed_wpe_kernel(const float* dx, int M, int T, int C, int Tb,
                                                        float* dwpe, int accumulate) {
  long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)Tb * C) return;
  int t = (int)(i / C), c = (int)(i % C);
  if (t >= T) {
    if (!accumulate) dwpe[i] = 0.f;
    return;
  }
  float s = 0.f;
  for (int m = t; m < M; m += T) s += dx[(long)m * C + c];
  dwpe[i] = accumulate ? dwpe[i] + s : s;
}

// ------------------------------------------------------------------ LayerNorm
// 4 consecutive act-type values at element offset o (o % 4 == 0).
__device__ __forceinline__ void store4(float* p, long o, float4 v) { *(float4*)(p + o) = v; }
__device__ __forceinline__ void store4(bf16_t* p, long o, float4 v) {
  *(uint2*)(p + o) = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
}
__device__ __forceinline__ float4 load4(const float* p, long o) { return *(const float4*)(p + o); }
__device__ __forceinline__ float4 load4(const bf16_t* p, long o) {
  uint2 u = *(const uint2*)(p + o);
  return make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y));
}

constexpr int LN_NV_MAX = 8;    // float4 vectors per lane -> C <= 2048
constexpr int LN_BWD_RPW = 4;   // rows per wave in the backward
constexpr int LN_BWD_RPB = 16;  // rows per workgroup in the backward

template <typename ActT, int LN_NV>
__global__ void __launch_bounds__(256) ln_fwd_kernel(const float* x, const float* w, const float* b,
                                                     int M, int C, float eps, ActT* y, float* mean,
                                                     float* rstd) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int C4 = C / 4;
  const float4* xr = (const float4*)(x + (long)row * C);
  float4 v[LN_NV];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < LN_NV; ++i) {
    int c = lane + 64 * i;
    v[i] = c < C4 ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  const float mu = warp_sum(s) / (float)C;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < LN_NV; ++i) {
    int c = lane + 64 * i;
    if (c < C4) {
      float a = v[i].x - mu, bb = v[i].y - mu, cc = v[i].z - mu, d = v[i].w - mu;
      q += (a * a + bb * bb) + (cc * cc + d * d);
    }
  }
  const float var = warp_sum(q) / (float)C;
  const float rs = 1.f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < LN_NV; ++i) {
    int c = lane + 64 * i;
    if (c < C4) {
      float4 ww = ((const float4*)w)[c];
      float4 bb = b ? ((const float4*)b)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      store4(y, (long)row * C + 4 * c,
             make_float4((v[i].x - mu) * rs * ww.x + bb.x, (v[i].y - mu) * rs * ww.y + bb.y,
                         (v[i].z - mu) * rs * ww.z + bb.z, (v[i].w - mu) * rs * ww.w + bb.w));
    }
  }
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

// dx = resid_in + rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat)), dxhat = dy * w.
// Per-workgroup partial sums of dy*xhat and dy go to partials[2][nblk][C].
template <typename ActT, int LN_NV>
__global__ void __launch_bounds__(256) ln_bwd_kernel(const ActT* dy, const float* x,
                                                     const float* mean, const float* rstd,
                                                     const float* w, const float* resid_in, int M,
                                                     int C, float* dx, ActT* dx_act,
                                                     float* partials) {
  extern __shared__ float sh[];  // [4 waves][2][C]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int C4 = C / 4;
  float4 aw[LN_NV], ab[LN_NV];
#pragma unroll
  for (int i = 0; i < LN_NV; ++i) aw[i] = ab[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int rr = 0; rr < LN_BWD_RPW; ++rr) {
    const int row = blockIdx.x * LN_BWD_RPB + wave * LN_BWD_RPW + rr;
    if (row >= M) break;
    const float mu = mean[row], rs = rstd[row];
    float4 xh[LN_NV], dh[LN_NV], g[LN_NV];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < LN_NV; ++i) {
      int c = lane + 64 * i;
      if (c < C4) {
        float4 xv = ((const float4*)(x + (long)row * C))[c];
        float4 ww = ((const float4*)w)[c];
        g[i] = load4(dy, (long)row * C + 4 * c);
        xh[i] = make_float4((xv.x - mu) * rs, (xv.y - mu) * rs, (xv.z - mu) * rs, (xv.w - mu) * rs);
        dh[i] = make_float4(g[i].x * ww.x, g[i].y * ww.y, g[i].z * ww.z, g[i].w * ww.w);
        s1 += (dh[i].x + dh[i].y) + (dh[i].z + dh[i].w);
        s2 += (dh[i].x * xh[i].x + dh[i].y * xh[i].y) + (dh[i].z * xh[i].z + dh[i].w * xh[i].w);
        aw[i].x += g[i].x * xh[i].x; aw[i].y += g[i].y * xh[i].y;
        aw[i].z += g[i].z * xh[i].z; aw[i].w += g[i].w * xh[i].w;
        ab[i].x += g[i].x; ab[i].y += g[i].y; ab[i].z += g[i].z; ab[i].w += g[i].w;
      }
    }
    const float c1 = warp_sum(s1) / (float)C, c2 = warp_sum(s2) / (float)C;
#pragma unroll
    for (int i = 0; i < LN_NV; ++i) {
      int c = lane + 64 * i;
      if (c < C4) {
        long o = (long)row * C + 4 * c;
        float4 r = resid_in ? ((const float4*)(resid_in + (long)row * C))[c]
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        float4 d = make_float4(r.x + rs * (dh[i].x - c1 - xh[i].x * c2),
                               r.y + rs * (dh[i].y - c1 - xh[i].y * c2),
                               r.z + rs * (dh[i].z - c1 - xh[i].z * c2),
                               r.w + rs * (dh[i].w - c1 - xh[i].w * c2));
        ((float4*)(dx + (long)row * C))[c] = d;
        store4(dx_act, o, d);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < LN_NV; ++i) {
    int c = lane + 64 * i;
    if (c < C4) {
      ((float4*)(sh + (wave * 2 + 0) * C))[c] = aw[i];
      ((float4*)(sh + (wave * 2 + 1) * C))[c] = ab[i];
    }
  }
  __syncthreads();
  const int nblk = gridDim.x;
  for (int c = threadIdx.x; c < C; c += 256) {
    float sw = ((sh[0 * C + c] + sh[2 * C + c]) + sh[4 * C + c]) + sh[6 * C + c];
    float sb = ((sh[1 * C + c] + sh[3 * C + c]) + sh[5 * C + c]) + sh[7 * C + c];
    partials[(long)blockIdx.x * C + c] = sw;
    partials[((long)nblk + blockIdx.x) * C + c] = sb;
  }
}

// out[c] (+)= sum over rows r of part[r, c], in two fixed-order stages.
// Stage 1: workgroup (x, y) owns 64 columns and rows [y*RS, (y+1)*RS); wave w
// sums rows w, w+4, ... of that slice and the four wave sums are added in wave
// order -> stage[y][c].  Stage 2 adds the RED_SLICES rows of `stage` in order.
constexpr int RED_SLICES = 16;
__global__ void __launch_bounds__(256) reduce_rows_stage1(const float* part, int R, int N,
                                                          float* stage) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  const int rs = (R + RED_SLICES - 1) / RED_SLICES;
  const int r0 = blockIdx.y * rs, r1 = min(R, r0 + rs);
  float s = 0.f;
  if (c < N) {
    int r = r0 + wave;
    for (; r + 12 < r1; r += 16) {  // four independent loads in flight
      float a = part[(long)r * N + c], b = part[(long)(r + 4) * N + c];
      float d = part[(long)(r + 8) * N + c], e = part[(long)(r + 12) * N + c];
      s += ((a + b) + d) + e;
    }
    for (; r < r1; r += 4) s += part[(long)r * N + c];
  }
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && c < N)
    stage[(long)blockIdx.y * N + c] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

__global__ void __launch_bounds__(256) reduce_rows_stage2(const float* stage, int N, float* out,
                                                          int accumulate) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= N || out == nullptr) return;
  float t = 0.f;
#pragma unroll
  for (int y = 0; y < RED_SLICES; ++y) t += stage[(long)y * N + c];
  out[c] = accumulate ? out[c] + t : t;
}

// `stage` holds RED_SLICES * N floats.
hipError_t reduce_rows(const float* part, int R, int N, float* out, int accumulate, float* stage,
                       hipStream_t s) {
  if (out == nullptr) return hipSuccess;
  reduce_rows_stage1<<<dim3((unsigned)cdiv(N, 64), RED_SLICES), 256, 0, s>>>(part, R, N, stage);
  reduce_rows_stage2<<<(unsigned)cdiv(N, 256), 256, 0, s>>>(stage, N, out, accumulate);
  return hipGetLastError();
}

// Column sums of an act matrix [M, N]: partial[chunk, n] over 64-row chunks.
// A wave covers 64 x (16 / sizeof) consecutive columns with 16-byte loads;
// the four waves of a workgroup take rows w, w+4, ... of the chunk and are
// added in wave order.
constexpr int CS_ROWS = 64;
template <typename ActT>
__global__ void __launch_bounds__(256) colsum_kernel(const ActT* x, int M, int N, float* partial) {
  constexpr int EPV = 16 / sizeof(ActT);
  __shared__ float red[4][64 * EPV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = (blockIdx.x * 64 + lane) * EPV;
  const int r0 = blockIdx.y * CS_ROWS, r1 = min(M, r0 + CS_ROWS);
  float acc[EPV];
#pragma unroll
  for (int k = 0; k < EPV; ++k) acc[k] = 0.f;
  if (n < N) {
    for (int r = r0 + wave; r < r1; r += 4) {
      u32x4 raw = *(const u32x4*)(x + (long)r * N + n);
      if constexpr (EPV == 8) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] += bf_lo(raw[k]);
          acc[2 * k + 1] += bf_hi(raw[k]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] += __uint_as_float(raw[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < EPV; ++k) red[wave][lane * EPV + k] = acc[k];
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * EPV; i += 256) {
    const int col = blockIdx.x * 64 * EPV + i;
    if (col < N)
      partial[(long)blockIdx.y * N + col] = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
  }
}

// ------------------------------------------------------------------ cross-entropy
// One workgroup per row; the whole row lives in registers, so the logits are
// read once and the gradient written once.  loss = lse_{v<V} z - z[tgt];
// z is overwritten by (softmax - onehot) / M on [0, V) and 0 on [V, ldz).
constexpr int CE_THREADS = 1024;
constexpr int CE_NV = 8;

template <typename ActT>
__global__ void __launch_bounds__(CE_THREADS) ce_kernel(ActT* z, int M, int V, int ldz,
                                                        const int32_t* tgt, float* loss_rows,
                                                        float inv_count) {
  constexpr int EPV = 16 / sizeof(ActT);
  __shared__ float red[CE_THREADS / 64];
  __shared__ float zt_s;
  const int row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  ActT* zr = z + (long)row * ldz;
  const int target = tgt[row];
  const int nvec = ldz / EPV;
  float v[CE_NV][EPV];
#pragma unroll
  for (int i = 0; i < CE_NV; ++i) {
    int vix = t + i * CE_THREADS;
    if (vix < nvec) {
      u32x4 raw = *(const u32x4*)(zr + (long)vix * EPV);
      const ActT* e = (const ActT*)&raw;
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        int col = vix * EPV + k;
        v[i][k] = col < V ? Act<ActT>::load(e, k) : -INFINITY;
      }
    } else {
#pragma unroll
      for (int k = 0; k < EPV; ++k) v[i][k] = -INFINITY;
    }
  }
  if (t == 0) zt_s = Act<ActT>::load(zr, target);
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < CE_NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) mx = fmaxf(mx, v[i][k]);
  mx = warp_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
  for (int i = 1; i < CE_THREADS / 64; ++i) mx = fmaxf(mx, red[i]);
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < CE_NV; ++i)
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
      float e = expf(v[i][k] - mx);
      v[i][k] = e;
      s += e;
    }
  s = warp_sum(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  s = 0.f;
  for (int i = 0; i < CE_THREADS / 64; ++i) s += red[i];
  const float inv_s = 1.f / s;
  if (t == 0) loss_rows[row] = (mx + logf(s)) - zt_s;
#pragma unroll
  for (int i = 0; i < CE_NV; ++i) {
    int vix = t + i * CE_THREADS;
    if (vix < nvec) {
      u32x4 raw;
      ActT* e = (ActT*)&raw;
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        int col = vix * EPV + k;
        float d = 0.f;
        if (col < V) d = (v[i][k] * inv_s - (col == target ? 1.f : 0.f)) * inv_count;
        Act<ActT>::store(e, k, d);
      }
      *(u32x4*)(zr + (long)vix * EPV) = raw;
    }
  }
}

__global__ void __launch_bounds__(1024) mean_kernel(const float* x, int n, float* out) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 1024) s += (double)x[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = (float)(red[0] / (double)n);
}

// ------------------------------------------------------------------ sum of squares
constexpr int SS_BLOCKS = 1024;
__global__ void __launch_bounds__(256) sumsq_kernel(const float* x, int64_t n, double* partials) {
  __shared__ double red[256];
  const int64_t chunk = ((n + SS_BLOCKS - 1) / SS_BLOCKS + 3) / 4 * 4;  // keeps float4 alignment
  const int64_t b = (int64_t)blockIdx.x * chunk, e = std::min<int64_t>(n, b + chunk);
  float s = 0.f;
  int64_t i = b + threadIdx.x * 4;
  for (; i + 3 < e; i += 1024) {
    float4 v = *(const float4*)(x + i);
    s += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
  }
  for (; i < e; ++i) s += x[i] * x[i];  // tail (only when the chunk is ragged)
  red[threadIdx.x] = (double)s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) partials[blockIdx.x] = red[0];
}

__global__ void __launch_bounds__(256) sum_partials_kernel(const double* partials, int n,
                                                           double* out) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) s += partials[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = red[0];
}

__global__ void __launch_bounds__(256) to_bf16_kernel(const float* x, int64_t n, bf16_t* y) {
  int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    float4 v = *(const float4*)(x + i);
    *(uint2*)(y + i) = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
  } else {
    for (; i < n; ++i) y[i] = f2bf(x[i]);
  }
}

}  // namespace

hipError_t embed_fwd(int prec, const int32_t* idx, const float* wte, const float* wpe, int M, int T,
                     int C, float* x, hipStream_t s) {
  (void)prec;
  long n = (long)M * (C / 4);
  if (n == 0) return hipSuccess;
  embed_fwd_kernel<<<(unsigned)cdiv(n, 256), 256, 0, s>>>(idx, wte, wpe, M, T, C, x);
  return hipGetLastError();
}

hipError_t embed_bwd(const int32_t* idx, const float* dx, int M, int T, int C, int Vp, int Tb,
                     float* dwte, int wte_accumulate, float* dwpe, int wpe_accumulate,
                     EmbedBwdScratch scr, hipStream_t s) {
  fill_i32<<<(unsigned)cdiv(Vp, 256), 256, 0, s>>>(scr.counts, Vp, 0);
  if (M > 0) embed_count_kernel<<<(unsigned)cdiv(M, 256), 256, 0, s>>>(idx, M, scr.counts);
  scan_kernel<<<1, 1024, 0, s>>>(scr.counts, Vp, scr.offsets);
  if (M > 0)
    embed_rank_kernel<<<(unsigned)cdiv(M, 256), 256, 0, s>>>(idx, M, scr.offsets, scr.perm);
  dim3 g((unsigned)Vp, (unsigned)cdiv(C, 256));
  embed_wte_kernel<<<g, 256, 0, s>>>(dx, C, scr.counts, scr.offsets, scr.perm, dwte,
                                     wte_accumulate);
  embed_wpe_kernel<<<(unsigned)cdiv((long)Tb * C, 256), 256, 0, s>>>(dx, M, T, C, Tb, dwpe,
                                                                     wpe_accumulate);
  return hipGetLastError();
}

hipError_t layernorm_fwd(int prec, const float* x, const float* w, const float* b, int M, int C,
                         float eps, void* y, float* mean, float* rstd, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (C % 4 || C > 4 * 64 * LN_NV_MAX) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)cdiv(M, 4);
  const int nv = (int)cdiv(C / 4, 64);  // float4 vectors per lane
#define LNF_(NV)                                                                                  \
  if (nv <= NV) {                                                                                 \
    if (prec == GPT_BF16)                                                                         \
      ln_fwd_kernel<bf16_t, NV><<<grid, 256, 0, s>>>(x, w, b, M, C, eps, (bf16_t*)y, mean, rstd); \
    else                                                                                          \
      ln_fwd_kernel<float, NV><<<grid, 256, 0, s>>>(x, w, b, M, C, eps, (float*)y, mean, rstd);   \
    return hipGetLastError();                                                                     \
  }
  LNF_(1) LNF_(2) LNF_(3) LNF_(4) LNF_(8)
#undef LNF_
  return hipErrorInvalidValue;
}

int layernorm_bwd_partial_rows(int M) { return (int)cdiv(M, LN_BWD_RPB); }
int64_t layernorm_bwd_partial_floats(int M, int C) {
  return (2L * layernorm_bwd_partial_rows(M) + RED_SLICES) * C;
}

hipError_t layernorm_bwd(int prec, const void* dy, const float* x, const float* mean,
                         const float* rstd, const float* w, const float* resid_in, int M, int C,
                         float* dx, void* dx_act, float* dw, float* db, int accumulate,
                         float* partials, hipStream_t s) {
  if (C % 4 || C > 4 * 64 * LN_NV_MAX) return hipErrorInvalidValue;
  const int nblk = layernorm_bwd_partial_rows(M);
  const int nv = (int)cdiv(C / 4, 64);
  if (nblk > 0) {
    const size_t shmem = (size_t)8 * C * sizeof(float);
    bool done = false;
#define LNB_(NV)                                                                                 \
  if (!done && nv <= NV) {                                                                       \
    if (prec == GPT_BF16)                                                                        \
      ln_bwd_kernel<bf16_t, NV><<<nblk, 256, shmem, s>>>((const bf16_t*)dy, x, mean, rstd, w,    \
                                                         resid_in, M, C, dx, (bf16_t*)dx_act,    \
                                                         partials);                              \
    else                                                                                         \
      ln_bwd_kernel<float, NV><<<nblk, 256, shmem, s>>>((const float*)dy, x, mean, rstd, w,      \
                                                        resid_in, M, C, dx, (float*)dx_act,      \
                                                        partials);                               \
    done = true;                                                                                 \
  }
    LNB_(1) LNB_(2) LNB_(3) LNB_(4) LNB_(8)
#undef LNB_
  }
  float* stage = partials + 2L * nblk * C;
  hipError_t e = reduce_rows(partials, nblk, C, dw, accumulate, stage, s);
  if (e != hipSuccess) return e;
  return reduce_rows(partials + (long)nblk * C, nblk, C, db, accumulate, stage, s);
}

int colsum_partial_rows(int M) { return (int)cdiv(M, CS_ROWS); }
int64_t colsum_partial_floats(int M, int N) { return ((long)colsum_partial_rows(M) + RED_SLICES) * N; }

hipError_t colsum(int prec, const void* x, int M, int N, float* out, int accumulate,
                  float* partials, hipStream_t s) {
  if (N % 8) return hipErrorInvalidValue;
  const int R = colsum_partial_rows(M);
  if (R > 0) {
    if (prec == GPT_BF16)
      colsum_kernel<bf16_t><<<dim3((unsigned)cdiv(N, 512), (unsigned)R), 256, 0, s>>>(
          (const bf16_t*)x, M, N, partials);
    else
      colsum_kernel<float><<<dim3((unsigned)cdiv(N, 256), (unsigned)R), 256, 0, s>>>(
          (const float*)x, M, N, partials);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return reduce_rows(partials, R, N, out, accumulate, partials + (long)R * N, s);
}

bool cross_entropy_supported(int prec, int ldz) {
  int epv = prec == GPT_BF16 ? 8 : 4;
  return ldz % epv == 0 && ldz <= CE_THREADS * CE_NV * epv;
}

hipError_t cross_entropy(int prec, void* logits, int M, int V, int ldz, const int32_t* tgt,
                         float* loss_rows, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (!cross_entropy_supported(prec, ldz) || V > ldz) return hipErrorInvalidValue;
  float inv = 1.f / (float)M;
  if (prec == GPT_BF16)
    ce_kernel<bf16_t><<<M, CE_THREADS, 0, s>>>((bf16_t*)logits, M, V, ldz, tgt, loss_rows, inv);
  else
    ce_kernel<float><<<M, CE_THREADS, 0, s>>>((float*)logits, M, V, ldz, tgt, loss_rows, inv);
  return hipGetLastError();
}

hipError_t mean_loss(const float* loss_rows, int M, float* out, hipStream_t s) {
  mean_kernel<<<1, 1024, 0, s>>>(loss_rows, M, out);
  return hipGetLastError();
}

hipError_t sumsq(const float* x, int64_t n, double* partials, double* out, hipStream_t s) {
  sumsq_kernel<<<SS_BLOCKS, 256, 0, s>>>(x, n, partials);
  sum_partials_kernel<<<1, 256, 0, s>>>(partials, SS_BLOCKS, out);
  return hipGetLastError();
}

hipError_t to_bf16(const float* x, int64_t n, uint16_t* y, hipStream_t s) {
  if (n == 0) return hipSuccess;
  to_bf16_kernel<<<(unsigned)cdiv(cdiv(n, 4), 256), 256, 0, s>>>(x, n, y);
  return hipGetLastError();
}

}  // namespace gpt
