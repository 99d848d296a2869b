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
// Ids outside [0, V) read row 0 and mark *flag = gen; ids_out[m] receives the
// id used (the backward's copy).
__global__ void __launch_bounds__(256) embed_fwd_kernel(const int32_t* idx, const float* wte,
                                                        const float* wpe, int M, int T, int C,
                                                        int V, float* x, int32_t* ids_out,
                                                        int32_t* flag, int32_t gen) {
  const int C4 = C / 4;
  long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)M * C4) return;
  int m = (int)(i / C4), c = (int)(i % C4);
  const int tok = checked_id(idx[m], V, flag, gen);
  if (c == 0 && ids_out) ids_out[m] = tok;
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

// Exclusive scan of counts[n] -> offsets[n] over tiles of 1024: scan_tiles
// writes each tile's total, scan_apply scans a tile (wave shuffles, then the
// wave totals) and adds the totals of the tiles before it.
__global__ void __launch_bounds__(1024) scan_tiles(const int32_t* counts, int n, int32_t* tsum) {
  __shared__ int32_t wsum[16];
  const int t = threadIdx.x, i = blockIdx.x * 1024 + t;
  int v = i < n ? counts[i] : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((t & 63) == 0) wsum[t >> 6] = v;
  __syncthreads();
  if (t == 0) {
    int s = 0;
    for (int w = 0; w < 16; ++w) s += wsum[w];
    tsum[blockIdx.x] = s;
  }
}

__global__ void __launch_bounds__(1024) scan_apply(const int32_t* counts, int n,
                                                   const int32_t* tsum, int32_t* offsets) {
  __shared__ int32_t wsum[16], before[16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, i = blockIdx.x * 1024 + t;
  // totals of the earlier tiles
  int b = 0;
  for (int k = t; k < (int)blockIdx.x; k += 1024) b += tsum[k];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) b += __shfl_xor(b, o, 64);
  if (lane == 0) before[wave] = b;
  const int c = i < n ? counts[i] : 0;
  int x = c;  // inclusive scan within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int acc = x - c;
  for (int w = 0; w < 16; ++w) acc += before[w] + (w < wave ? wsum[w] : 0);
  if (i < n) offsets[i] = acc;
}

// rank[p] += #{p' < p in block y : idx[p'] == idx[p]} for p in block x (256
// positions per block, y <= x).  Integer atomics: exact in any order.
__global__ void __launch_bounds__(256) embed_rank_kernel(const int32_t* __restrict__ idx, int M,
                                                         int32_t* __restrict__ rank) {
  const int bx = blockIdx.x, by = blockIdx.y;
  if (by > bx) return;
  __shared__ int32_t tile[256];
  const int q = by * 256 + threadIdx.x;
  tile[threadIdx.x] = q < M ? idx[q] : -1;
  __syncthreads();
  const int p = bx * 256 + threadIdx.x;
  if (p >= M) return;
  const int mine = idx[p];
  const int lim = by < bx ? 256 : (int)threadIdx.x;
  int r = 0;
  for (int k = 0; k < lim; ++k) r += tile[k] == mine;
  if (r) atomicAdd(&rank[p], r);
}

// perm[offsets[idx[p]] + rank[p]] = p: positions grouped by token, increasing
// within a token (a stable counting sort).
__global__ void embed_place_kernel(const int32_t* idx, int M, const int32_t* offsets,
                                   const int32_t* rank, int32_t* perm) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p < M) perm[offsets[idx[p]] + rank[p]] = p;
}

// dwte rows from the sorted positions: workgroup ch sums its EB_CHUNK sorted
// entries segment by segment (a segment = the positions of one token), in
// position order.  A segment wholly inside the chunk is added to dwte; the
// fragment of a segment that began in an earlier chunk goes to carry_first[ch]
// (flag EB_SPAN when it also continues past the chunk), the fragment of one
// that began here and continues goes to carry_last[ch] (flag EB_LAST).
constexpr int EB_CHUNK = 16;
constexpr int EB_LAST = 1, EB_SPAN = 2;

__global__ void __launch_bounds__(256) embed_chunk_kernel(
    const float* __restrict__ dx, int M, int C, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, float* __restrict__ dwte, float* __restrict__ carry_first,
    float* __restrict__ carry_last, int32_t* __restrict__ flags, int32_t* __restrict__ last_tok) {
  __shared__ int32_t pos[EB_CHUNK], tok[EB_CHUNK];
  __shared__ int32_t nb[2];  // tokens of the entries just before and after the chunk
  const int ch = blockIdx.x;
  const int i0 = ch * EB_CHUNK, n = min(M - i0, EB_CHUNK);
  if (threadIdx.x < n) {
    const int pp = perm[i0 + threadIdx.x];
    pos[threadIdx.x] = pp;
    tok[threadIdx.x] = idx[pp];
  }
  if (threadIdx.x == 64) nb[0] = i0 > 0 ? idx[perm[i0 - 1]] : -1;
  if (threadIdx.x == 65) nb[1] = i0 + n < M ? idx[perm[i0 + n]] : -1;
  __syncthreads();
  const bool first_cont = nb[0] == tok[0];     // first segment began in an earlier chunk
  const bool last_cont = nb[1] == tok[n - 1];  // last segment continues past the chunk
  const bool one_token = tok[0] == tok[n - 1];
  if (threadIdx.x == 0) {
    flags[ch] = (last_cont && !(first_cont && one_token) ? EB_LAST : 0) |
                (first_cont && last_cont && one_token ? EB_SPAN : 0);
    last_tok[ch] = tok[n - 1];
  }
  const int C4 = C / 4;
  for (int c = threadIdx.x; c < C4; c += 256) {
    float4 v[EB_CHUNK];  // all rows in flight at once
#pragma unroll
    for (int i = 0; i < EB_CHUNK; ++i)
      if (i < n) v[i] = ((const float4*)(dx + (long)pos[i] * C))[c];
    float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < EB_CHUNK; ++i) {
      if (i < n) {
        run.x += v[i].x; run.y += v[i].y; run.z += v[i].z; run.w += v[i].w;
        if (i + 1 == n || tok[i + 1] != tok[i]) {  // segment ends at entry i
          if (first_cont && tok[i] == tok[0]) {
            ((float4*)(carry_first + (long)ch * C))[c] = run;
          } else if (i + 1 == n && last_cont) {
            ((float4*)(carry_last + (long)ch * C))[c] = run;
          } else {
            float4* o = (float4*)(dwte + (long)tok[i] * C) + c;
            const float4 a = *o;
            *o = make_float4(a.x + run.x, a.y + run.y, a.z + run.z, a.w + run.w);
          }
          run = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
  }
}

// Segments that cross chunk boundaries: the chunk where one begins (EB_LAST)
// finds the chunk where it ends (the first later chunk without EB_SPAN), then
// adds its own fragment and those of the following chunks in order.
__global__ void __launch_bounds__(256) embed_carry_kernel(int C, int nch,
                                                          const float* __restrict__ carry_first,
                                                          const float* __restrict__ carry_last,
                                                          const int32_t* __restrict__ flags,
                                                          const int32_t* __restrict__ last_tok,
                                                          float* __restrict__ dwte) {
  __shared__ int end_s;
  const int ch = blockIdx.x;
  if (!(flags[ch] & EB_LAST)) return;
  if (threadIdx.x == 0) end_s = nch;
  __syncthreads();
  for (int base = ch + 1; base < nch; base += 256) {
    const int k = base + threadIdx.x;
    if (k < nch && !(flags[k] & EB_SPAN)) atomicMin(&end_s, k);
    __syncthreads();
    const bool found = end_s < nch;
    __syncthreads();  // every thread has read end_s before the next round may lower it
    if (found) break;
  }
  const int e = min(end_s, nch - 1);
  const int v = last_tok[ch];
  const int C4 = C / 4;
  for (int c = threadIdx.x; c < C4; c += 256) {
    float4 s = ((const float4*)(carry_last + (long)ch * C))[c];
#pragma unroll 8
    for (int k = ch + 1; k <= e; ++k) {
      const float4 f = ((const float4*)(carry_first + (long)k * C))[c];
      s.x += f.x; s.y += f.y; s.z += f.z; s.w += f.w;
    }
    float4* o = (float4*)(dwte + (long)v * C) + c;
    const float4 a = *o;
    *o = make_float4(a.x + s.x, a.y + s.y, a.z + s.z, a.w + s.w);
  }
}

__global__ void fill_f32(float* p, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
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

// ------------------------------------------------------------------ seeded init
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of two 32x32 -> 64-bit products on
// words 0 and 2, the new block (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^
// k1, lo(M0 c0)), the key bumped by the Weyl increments between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1,
                   (uint32_t)p0);
  }
  return c;
}

// p[i - begin] for flat indices i in [begin, begin + n): std * z(i) for the
// first n_normal of them, 0 after.  z(i): block j = i / 4 of Philox (counter
// (j lo, j hi, 0, 0), key (seed lo, seed hi)); words (x0, x1) -> z(4j), z(4j+1)
// and (x2, x3) -> z(4j+2), z(4j+3) by Box-Muller (Box and Muller, 1958) in
// double: r = sqrt(-2 ln((x + 1) / 2^32)), angle 2 pi x' / 2^32.
__global__ void __launch_bounds__(256) init_normal_kernel(float* __restrict__ p, int64_t begin,
                                                          int64_t n, int64_t n_normal, double stdv,
                                                          uint64_t seed) {
  const int64_t j = begin / 4 + (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (4 * j >= begin + n) return;
  const uint4 x = philox4x32_10(make_uint4((uint32_t)j, (uint32_t)((uint64_t)j >> 32), 0u, 0u),
                                (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  double z[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const double r = sqrt(-2.0 * log(((double)w[2 * h] + 1.0) * 0x1p-32));
    double sn, cs;
    sincos(6.283185307179586 * ((double)w[2 * h + 1] * 0x1p-32), &sn, &cs);
    z[2 * h] = r * cs;
    z[2 * h + 1] = r * sn;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t i = 4 * j + q;
    if (i < begin || i >= begin + n) continue;
    p[i - begin] = i - begin < n_normal ? (float)(stdv * z[q]) : 0.f;
  }
}

__global__ void __launch_bounds__(256) fill_value_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
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
constexpr int LN_BWD_RPB = 64;  // rows per workgroup in the backward (16 waves)

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
// A workgroup of LN_BWD_WAVES waves owns LN_BWD_RPB rows (LN_BWD_RPW per
// wave).  Its partial sums of dy*xhat and dy go to partials[2][nblk][C]: the
// wave sums are combined in LDS in four rounds of four waves, in wave order.
constexpr int LN_BWD_WAVES = 16;
template <typename ActT, int LN_NV>
__global__ void __launch_bounds__(64 * LN_BWD_WAVES) ln_bwd_kernel(
    const ActT* dy, const float* x, const float* mean, const float* rstd, const float* w,
    const float* resid_in, int M, int C, float* dx, ActT* dx_act, float* partials) {
  extern __shared__ float sh[];  // [4 slots][2][C]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int C4 = C / 4;
  float4 aw[LN_NV], ab[LN_NV];
#pragma unroll
  for (int i = 0; i < LN_NV; ++i) aw[i] = ab[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int rr = 0; rr < LN_BWD_RPW; ++rr) {
    const int row = blockIdx.x * LN_BWD_RPB + wave * LN_BWD_RPW + rr;
    if (row >= M) break;
    const float mu = mean[row], rs = rstd[row];
    float4 xh[LN_NV], dh[LN_NV], r[LN_NV];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < LN_NV; ++i) {
      const int c = lane + 64 * i;
      if (c < C4) {
        const float4 xv = ((const float4*)(x + (long)row * C))[c];
        const float4 ww = ((const float4*)w)[c];
        const float4 g = load4(dy, (long)row * C + 4 * c);
        r[i] = resid_in ? ((const float4*)(resid_in + (long)row * C))[c]
                        : make_float4(0.f, 0.f, 0.f, 0.f);
        xh[i] = make_float4((xv.x - mu) * rs, (xv.y - mu) * rs, (xv.z - mu) * rs, (xv.w - mu) * rs);
        dh[i] = make_float4(g.x * ww.x, g.y * ww.y, g.z * ww.z, g.w * ww.w);
        s1 += (dh[i].x + dh[i].y) + (dh[i].z + dh[i].w);
        s2 += (dh[i].x * xh[i].x + dh[i].y * xh[i].y) + (dh[i].z * xh[i].z + dh[i].w * xh[i].w);
        aw[i].x += g.x * xh[i].x; aw[i].y += g.y * xh[i].y;
        aw[i].z += g.z * xh[i].z; aw[i].w += g.w * xh[i].w;
        ab[i].x += g.x; ab[i].y += g.y; ab[i].z += g.z; ab[i].w += g.w;
      }
    }
    const float c1 = warp_sum(s1) / (float)C, c2 = warp_sum(s2) / (float)C;
#pragma unroll
    for (int i = 0; i < LN_NV; ++i) {
      const int c = lane + 64 * i;
      if (c < C4) {
        const long o = (long)row * C + 4 * c;
        const float4 d = make_float4(r[i].x + rs * (dh[i].x - c1 - xh[i].x * c2),
                                     r[i].y + rs * (dh[i].y - c1 - xh[i].y * c2),
                                     r[i].z + rs * (dh[i].z - c1 - xh[i].z * c2),
                                     r[i].w + rs * (dh[i].w - c1 - xh[i].w * c2));
        *(float4*)(dx + o) = d;
        store4(dx_act, o, d);
      }
    }
  }
  // waves 4k .. 4k+3 add into slots 0..3 in round k
  float* slot = sh + (wave & 3) * 2 * C;
  for (int round = 0; round < LN_BWD_WAVES / 4; ++round) {
    if ((wave >> 2) == round) {
#pragma unroll
      for (int i = 0; i < LN_NV; ++i) {
        const int c = lane + 64 * i;
        if (c < C4) {
          float4* pw = (float4*)slot + c;
          float4* pb = (float4*)(slot + C) + c;
          if (round == 0) {
            *pw = aw[i];
            *pb = ab[i];
          } else {
            const float4 a = *pw, b = *pb;
            *pw = make_float4(a.x + aw[i].x, a.y + aw[i].y, a.z + aw[i].z, a.w + aw[i].w);
            *pb = make_float4(b.x + ab[i].x, b.y + ab[i].y, b.z + ab[i].z, b.w + ab[i].w);
          }
        }
      }
    }
    __syncthreads();
  }
  const int nblk = gridDim.x;
  for (int c = threadIdx.x; c < C; c += 64 * LN_BWD_WAVES) {
    float sw = ((sh[0 * C + c] + sh[2 * C + c]) + sh[4 * C + c]) + sh[6 * C + c];
    float sb = ((sh[1 * C + c] + sh[3 * C + c]) + sh[5 * C + c]) + sh[7 * C + c];
    partials[(long)blockIdx.x * C + c] = sw;
    partials[((long)nblk + blockIdx.x) * C + c] = sb;
  }
}

// out_p[c] (+)= sum over rows r of part[p * R * N + r * N + c] for parts
// p = blockIdx.y, in a fixed order: workgroup (x, p) owns 64 columns; wave w
// of 16 sums rows w, w + 16, ... (four loads in flight) and the 16 wave sums
// are added in wave order.
__global__ void __launch_bounds__(1024) colreduce_kernel(const float* __restrict__ part, int R,
                                                         int N, float* out0, float* out1,
                                                         int accumulate) {
  __shared__ float red[16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  const float* pp = part + (long)blockIdx.y * R * N;
  float* out = blockIdx.y ? out1 : out0;
  float s = 0.f;
  if (c < N) {
    int r = wave;
    for (; r + 48 < R; r += 64) {
      const float a = pp[(long)r * N + c], b = pp[(long)(r + 16) * N + c];
      const float d = pp[(long)(r + 32) * N + c], e = pp[(long)(r + 48) * N + c];
      s += ((a + b) + d) + e;
    }
    for (; r < R; r += 16) s += pp[(long)r * N + c];
  }
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && c < N && out) {
    float t = red[0][lane];
#pragma unroll
    for (int w = 1; w < 16; ++w) t += red[w][lane];
    out[c] = accumulate ? out[c] + t : t;
  }
}

// One or two column reductions of R x N partial rows (part, then part + R * N).
hipError_t reduce_rows(const float* part, int R, int N, float* out0, float* out1, int accumulate,
                       hipStream_t s) {
  if (out0 == nullptr && out1 == nullptr) return hipSuccess;
  const unsigned parts = out1 ? 2 : 1;
  colreduce_kernel<<<dim3((unsigned)cdiv(N, 64), parts), 1024, 0, s>>>(part, R, N, out0, out1,
                                                                       accumulate);
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
// read once and the gradient written once (fp32: the generic kernel, bf16:
// ce_bf16_kernel).  loss = lse_{v<V} z - z[tgt];
// z is overwritten by (softmax - onehot) / M on [0, V) and 0 on [V, ldz).
constexpr int CE_THREADS = 1024;
constexpr int CE_NV = 8;
constexpr float LOG2E_F = 1.4426950408889634f;

template <typename ActT>
__global__ void __launch_bounds__(CE_THREADS) ce_kernel(ActT* z, int M, int V, int ldz,
                                                        const int32_t* tgt, float* loss_rows,
                                                        float inv_count, int32_t* flag,
                                                        int32_t gen) {
  constexpr int EPV = 16 / sizeof(ActT);
  __shared__ float red[CE_THREADS / 64];
  __shared__ float zt_s;
  const int row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  ActT* zr = z + (long)row * ldz;
  const int target = checked_id(tgt[row], V, t == 0 ? flag : nullptr, gen);
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

// bf16 rows: the logits stay in registers as packed bf16 (4 VGPRs per 8
// values, so two rows fit per CU), each thread reduces its values to a
// (max, sum of exp) pair and one block reduction combines the pairs in a fixed
// order.  exp(x - m) is evaluated as exp2(x log2 e - m log2 e).
__device__ __forceinline__ void lse_combine(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  const float a = m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - mn) * LOG2E_F);
  const float b = m2 == -INFINITY ? 0.f : s2 * __builtin_amdgcn_exp2f((m2 - mn) * LOG2E_F);
  m = mn;
  s = a + b;
}

__global__ void __launch_bounds__(CE_THREADS, 8) ce_bf16_kernel(bf16_t* z, int V, int ldz,
                                                             const int32_t* tgt,
                                                             float* loss_rows, float inv_count,
                                                             int32_t* flag, int32_t gen) {
  __shared__ float red_m[CE_THREADS / 64], red_s[CE_THREADS / 64];
  const int row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  bf16_t* zr = z + (long)row * ldz;
  const int target = checked_id(tgt[row], V, t == 0 ? flag : nullptr, gen);
  const int nvec = ldz / 8;
  u32x4 raw[CE_NV];
#pragma unroll
  for (int i = 0; i < CE_NV; ++i) {
    const int vix = t + i * CE_THREADS;
    raw[i] = vix < nvec ? *(const u32x4*)(zr + (long)vix * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  float zt = 0.f;
  if (t == 0) zt = bf2f(zr[target]);
  // running (max, sum) over this thread's vectors, one vector at a time, so
  // only the packed row stays live
  // (columns at or past V, the vocabulary padding, count as -inf)
  float mx = -INFINITY, sum = 0.f;
#pragma unroll
  for (int i = 0; i < CE_NV; ++i) {
    const int lim = V - (t + i * CE_THREADS) * 8;  // valid values in this vector
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float v = (k & 1) ? bf_hi(raw[i][k >> 1]) : bf_lo(raw[i][k >> 1]);
      x[k] = k < lim ? v : -INFINITY;
    }
    float vm = x[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) vm = fmaxf(vm, x[k]);
    lse_combine(mx, sum, vm, 0.f);
    if (mx != -INFINITY) {
      const float ml = mx * LOG2E_F;
      float vs = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) vs += __builtin_amdgcn_exp2f(fmaf(x[k], LOG2E_F, -ml));
      sum += vs;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(mx, o, 64), s2 = __shfl_xor(sum, o, 64);
    lse_combine(mx, sum, m2, s2);
  }
  if (lane == 0) {
    red_m[wave] = mx;
    red_s[wave] = sum;
  }
  __syncthreads();
  mx = red_m[0];
  sum = red_s[0];
  for (int w = 1; w < CE_THREADS / 64; ++w) lse_combine(mx, sum, red_m[w], red_s[w]);
  if (t == 0) loss_rows[row] = (mx + logf(sum)) - zt;
  const float inv_s = 1.f / sum, ml = mx * LOG2E_F;
  // Unpack again below instead of keeping 8 floats per vector alive across
  // the reduction (the empty asm hides that raw is unchanged).
#pragma unroll
  for (int i = 0; i < CE_NV; ++i) asm volatile("" : "+v"(raw[i]));
  int t2 = t;  // likewise the store addresses are recomputed
  asm volatile("" : "+v"(t2));
#pragma unroll
  for (int i = 0; i < CE_NV; ++i) {
    const int vix = t2 + i * CE_THREADS;
    if (vix < nvec) {
      float d[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int col = vix * 8 + k;
        const float x = (k & 1) ? bf_hi(raw[i][k >> 1]) : bf_lo(raw[i][k >> 1]);
        const float p = __builtin_amdgcn_exp2f(fmaf(x, LOG2E_F, -ml)) * inv_s;
        d[k] = col < V ? (p - (col == target ? 1.f : 0.f)) * inv_count : 0.f;
      }
      *(u32x4*)(zr + (long)vix * 8) = u32x4{pack_bf2(d[0], d[1]), pack_bf2(d[2], d[3]),
                                            pack_bf2(d[4], d[5]), pack_bf2(d[6], d[7])};
    }
  }
}

// The mean of x[n] in double, fixed order; NaN when *flag == gen (a token id
// of this forward was out of range).
__global__ void __launch_bounds__(1024) mean_kernel(const float* x, int n, float* out,
                                                    const int32_t* flag, int32_t gen) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 1024) s += (double)x[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const bool bad = flag != nullptr && *(volatile const int32_t*)flag == gen;
    out[0] = bad ? __builtin_nanf("") : (float)(red[0] / (double)n);
  }
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

// The same for many partials: 1024 threads, each summing every 1024th partial
// into four accumulators in turn (independent loads in flight), combined in a
// fixed order, then a fixed tree over the threads.
__global__ void __launch_bounds__(1024) sum_partials_wide_kernel(const double* partials, int n,
                                                                 double* out) {
  __shared__ double red[1024];
  double a[4] = {0.0, 0.0, 0.0, 0.0};
  int i = threadIdx.x;
  for (; i + 3 * 1024 < n; i += 4 * 1024) {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] += partials[i + k * 1024];
  }
  for (int k = 0; i < n; i += 1024, ++k) a[k] += partials[i];
  red[threadIdx.x] = (a[0] + a[1]) + (a[2] + a[3]);
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
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
                     int C, int V, float* x, int32_t* ids_out, int32_t* flag, int32_t gen,
                     hipStream_t s) {
  (void)prec;
  long n = (long)M * (C / 4);
  if (n == 0) return hipSuccess;
  embed_fwd_kernel<<<(unsigned)cdiv(n, 256), 256, 0, s>>>(idx, wte, wpe, M, T, C, V, x, ids_out,
                                                          flag, gen);
  return hipGetLastError();
}

int embed_bwd_chunks(int M) { return (int)cdiv(M, EB_CHUNK); }

hipError_t embed_bwd(const int32_t* idx, const float* dx, int M, int T, int C, int Vp, int Tb,
                     float* dwte, int wte_accumulate, float* dwpe, int wpe_accumulate,
                     EmbedBwdScratch scr, hipStream_t s) {
  if (!wte_accumulate)
    fill_f32<<<(unsigned)cdiv((long)Vp * C, 256), 256, 0, s>>>(dwte, (long)Vp * C);
  if (M > 0) {
    const int nb = (int)cdiv(M, 256), nch = embed_bwd_chunks(M);
    fill_i32<<<(unsigned)cdiv(Vp, 256), 256, 0, s>>>(scr.counts, Vp, 0);
    fill_i32<<<(unsigned)nb, 256, 0, s>>>(scr.rank, M, 0);
    embed_count_kernel<<<(unsigned)nb, 256, 0, s>>>(idx, M, scr.counts);
    const unsigned ntiles = (unsigned)cdiv(Vp, 1024);
    scan_tiles<<<ntiles, 1024, 0, s>>>(scr.counts, Vp, scr.tile_sums);
    scan_apply<<<ntiles, 1024, 0, s>>>(scr.counts, Vp, scr.tile_sums, scr.offsets);
    embed_rank_kernel<<<dim3((unsigned)nb, (unsigned)nb), 256, 0, s>>>(idx, M, scr.rank);
    embed_place_kernel<<<(unsigned)nb, 256, 0, s>>>(idx, M, scr.offsets, scr.rank, scr.perm);
    embed_chunk_kernel<<<(unsigned)nch, 256, 0, s>>>(dx, M, C, idx, scr.perm, dwte,
                                                     scr.carry_first, scr.carry_last, scr.flags,
                                                     scr.last_tok);
    embed_carry_kernel<<<(unsigned)nch, 256, 0, s>>>(C, nch, scr.carry_first, scr.carry_last,
                                                     scr.flags, scr.last_tok, dwte);
  }
  embed_wpe_kernel<<<(unsigned)cdiv((long)Tb * C, 256), 256, 0, s>>>(dx, M, T, C, Tb, dwpe,
                                                                     wpe_accumulate);
  return hipGetLastError();
}

hipError_t init_normal(float* p, int64_t begin, int64_t n, int64_t n_normal, double stdv,
                       uint64_t seed, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = cdiv((begin + n + 3) / 4 - begin / 4, 256);
  init_normal_kernel<<<(unsigned)blocks, 256, 0, s>>>(p, begin, n, n_normal, stdv, seed);
  return hipGetLastError();
}

hipError_t fill_value(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_value_kernel<<<(unsigned)cdiv(n, 256), 256, 0, s>>>(p, n, v);
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
  return 2L * layernorm_bwd_partial_rows(M) * C;
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
      ln_bwd_kernel<bf16_t, NV><<<nblk, 1024, shmem, s>>>((const bf16_t*)dy, x, mean, rstd, w,   \
                                                         resid_in, M, C, dx, (bf16_t*)dx_act,    \
                                                         partials);                              \
    else                                                                                         \
      ln_bwd_kernel<float, NV><<<nblk, 1024, shmem, s>>>((const float*)dy, x, mean, rstd, w,     \
                                                        resid_in, M, C, dx, (float*)dx_act,      \
                                                        partials);                               \
    done = true;                                                                                 \
  }
    LNB_(1) LNB_(2) LNB_(3) LNB_(4) LNB_(8)
#undef LNB_
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dw == nullptr) return hipSuccess;
  return reduce_rows(partials, nblk, C, dw, db, accumulate, s);
}

int colsum_partial_rows(int M) { return (int)cdiv(M, CS_ROWS); }
int64_t colsum_partial_floats(int M, int N) { return (long)colsum_partial_rows(M) * N; }

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
  return reduce_rows(partials, R, N, out, nullptr, accumulate, s);
}

bool cross_entropy_supported(int prec, int ldz) {
  int epv = prec == GPT_BF16 ? 8 : 4;
  return ldz % epv == 0 && ldz <= CE_THREADS * CE_NV * epv;
}

hipError_t cross_entropy(int prec, void* logits, int M, int V, int ldz, const int32_t* tgt,
                         float* loss_rows, int32_t* flag, int32_t gen, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (!cross_entropy_supported(prec, ldz) || V > ldz) return hipErrorInvalidValue;
  float inv = 1.f / (float)M;
  if (prec == GPT_BF16)
    ce_bf16_kernel<<<M, CE_THREADS, 0, s>>>((bf16_t*)logits, V, ldz, tgt, loss_rows, inv, flag,
                                            gen);
  else
    ce_kernel<float><<<M, CE_THREADS, 0, s>>>((float*)logits, M, V, ldz, tgt, loss_rows, inv,
                                              flag, gen);
  return hipGetLastError();
}

hipError_t mean_loss(const float* loss_rows, int M, float* out, const int32_t* flag, int32_t gen,
                     hipStream_t s) {
  mean_kernel<<<1, 1024, 0, s>>>(loss_rows, M, out, flag, gen);
  return hipGetLastError();
}

// Sums of squares over a table of ranges (begin, length, first block): block
// b belongs to the last range whose first block is <= b and sums its chunk of
// SQR_CHUNK elements of that range.
constexpr int64_t SQR_CHUNK = 256 * 64;
__global__ void __launch_bounds__(256) sumsq_ranges_kernel(const float* __restrict__ x,
                                                           const int64_t* __restrict__ rg,
                                                           int nr, double* partials) {
  __shared__ double red[256];
  int lo = 0, hi = nr - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (rg[3 * mid + 2] <= (int64_t)blockIdx.x) lo = mid; else hi = mid - 1;
  }
  const int64_t b = rg[3 * lo] + ((int64_t)blockIdx.x - rg[3 * lo + 2]) * SQR_CHUNK;
  const int64_t e = std::min<int64_t>(rg[3 * lo] + rg[3 * lo + 1], b + SQR_CHUNK);
  float s = 0.f;
  if ((rg[3 * lo] & 3) == 0) {  // 16-byte vectors (chunks start on a multiple of 4)
    const int64_t e4 = b + (e - b) / 4 * 4;
#pragma unroll 4
    for (int64_t i = b + threadIdx.x * 4; i < e4; i += 1024) {
      const float4 v = *(const float4*)(x + i);
      s += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
    }
    if ((int64_t)threadIdx.x < e - e4) s += x[e4 + threadIdx.x] * x[e4 + threadIdx.x];
  } else {
    for (int64_t i = b + threadIdx.x; i < e; i += 256) s += x[i] * x[i];
  }
  red[threadIdx.x] = (double)s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) partials[blockIdx.x] = red[0];
}

int sumsq_range_blocks(int64_t len) { return (int)std::max<int64_t>(1, (len + SQR_CHUNK - 1) / SQR_CHUNK); }

hipError_t sumsq_ranges(const float* x, const int64_t* d_ranges, int nranges, int blocks,
                        double* partials, hipStream_t s) {
  if (nranges < 1 || blocks < 1) return hipErrorInvalidValue;
  sumsq_ranges_kernel<<<(unsigned)blocks, 256, 0, s>>>(x, d_ranges, nranges, partials);
  return hipGetLastError();
}

hipError_t sum_partials(const double* partials, int n, double* out, hipStream_t s) {
  sum_partials_wide_kernel<<<1, 1024, 0, s>>>(partials, n, out);
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
