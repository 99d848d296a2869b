// Generation with a key/value cache: the kernels of one decode step that the
// training step does not have (nanoGPT README, "sampling / inference":
// sample.py continues a prompt token by token; llm.c summary, "Sampling").
//
//   gen_embed      x[b] = wte[token[b]] + wpe[pos]
//   attn_decode    one query per (sequence, head) against the cached keys and
//                  values 0..pos-1 plus its own (written to the cache here),
//                  running softmax per lane, merged in a fixed order (fp32:
//                  one key per thread; bf16: HD / 8 lanes per key, 16 waves)
//   sample         temperature / top-k / inverse-CDF draw per sequence (one
//                  1024-thread block per row): the top-k threshold by a 4-pass
//                  radix select on order-preserving keys, the cumulative sum by
//                  a fixed-order scan of per-thread chunks, so the same logits
//                  and u always give the same token
//   rows_linear    the bf16 matrix products of the step on MFMA 16x16x32, all
//                  of K in one workgroup (fp32 runs the training GEMM on B rows)

#include "common.h"
#include "kernels.h"

#include <cfloat>

namespace gpt {

namespace {

__global__ void __launch_bounds__(256) gen_embed_kernel(const int32_t* __restrict__ tok,
                                                        const float* __restrict__ wte,
                                                        const float* __restrict__ wpe,
                                                        const int32_t* __restrict__ pos_ptr,
                                                        int C, int V, float* __restrict__ x) {
  const int b = blockIdx.x;
  const int pos = *pos_ptr;
  const long t = checked_id(tok[b], V, nullptr, 0);  // out-of-range ids read row 0
  for (int c = threadIdx.x * 4; c < C; c += 256 * 4) {  // C % 64 == 0
    const float4 e = *(const float4*)(wte + t * C + c);
    const float4 p = *(const float4*)(wpe + (long)pos * C + c);
    *(float4*)(x + (long)b * C + c) = make_float4(e.x + p.x, e.y + p.y, e.z + p.z, e.w + p.w);
  }
}

constexpr int AD_THREADS = 256;

template <typename ActT, int HD>
__global__ void __launch_bounds__(AD_THREADS) attn_decode_kernel(
    const ActT* __restrict__ qkv, ActT* __restrict__ kc, ActT* __restrict__ vc,
    const int32_t* __restrict__ pos_ptr, int Tmax, int H, int left, float scale,
    ActT* __restrict__ out) {
  const int pos = *pos_ptr;
  __shared__ float q[HD];
  __shared__ float red[AD_THREADS];
  __shared__ float part[AD_THREADS][33];
  const int bh = blockIdx.x, b = bh / H, h = bh - b * H;
  const int C = H * HD, tid = threadIdx.x;
  const ActT* row = qkv + (long)b * 3 * C;
  ActT* kb = kc + (long)bh * Tmax * HD;
  ActT* vb = vc + (long)bh * Tmax * HD;
  if (tid < HD) {
    q[tid] = Act<ActT>::load(row, h * HD + tid) * scale;
    // this position's key and value join the cache
    Act<ActT>::store(kb, (long)pos * HD + tid, Act<ActT>::load(row, C + h * HD + tid));
    Act<ActT>::store(vb, (long)pos * HD + tid, Act<ActT>::load(row, 2 * C + h * HD + tid));
  }
  __syncthreads();
  const int j0 = left < 0 ? 0 : max(0, pos - left);
  float m = -FLT_MAX, l = 0.f, o[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) o[d] = 0.f;
  for (int j = j0 + tid; j <= pos; j += AD_THREADS) {
    // the current position reads its own key / value from qkv (the cache row
    // was written by this block above; reading qkv avoids relying on it)
    const ActT* kr = j == pos ? row + C + h * HD : kb + (long)j * HD;
    const ActT* vr = j == pos ? row + 2 * C + h * HD : vb + (long)j * HD;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < HD; ++d) s += q[d] * Act<ActT>::load(kr, d);
    const float mn = fmaxf(m, s);
    const float corr = __expf(m - mn), p = __expf(s - mn);
    l = l * corr + p;
#pragma unroll
    for (int d = 0; d < HD; ++d) o[d] = o[d] * corr + p * Act<ActT>::load(vr, d);
    m = mn;
  }
  // block max, then every thread's share rescaled to it
  red[tid] = m;
  __syncthreads();
  for (int w = AD_THREADS / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  const float f = l > 0.f ? __expf(m - M) : 0.f;
  red[tid] = l * f;
  __syncthreads();
  for (int w = AD_THREADS / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float L = red[0];
  // o summed over threads, 32 dimensions at a time, each column in thread order
#pragma unroll
  for (int d0 = 0; d0 < HD; d0 += 32) {
#pragma unroll
    for (int d = 0; d < 32; ++d) part[tid][d] = o[d0 + d] * f;
    __syncthreads();
    if (tid < 32) {
      float acc = 0.f;
      for (int t = 0; t < AD_THREADS; ++t) acc += part[t][tid];
      Act<ActT>::store(out, (long)b * C + h * HD + d0 + tid, acc / L);
    }
    __syncthreads();
  }
}

// bf16 decode attention, one 1024-thread workgroup per (sequence, head).
// HD / 8 lanes share a key, each holding 8 of its dimensions (one 16-byte
// load of the key row and one of the value row), so a wave reads 64 / (HD / 8)
// whole rows per load; wave w takes key blocks w, w + 16, ... and issues the
// loads of AW_DEPTH blocks before using them.  A lane keeps a running softmax
// over its keys; the lanes of a wave merge by a fixed xor butterfly (every
// lane ends with the same total), the 16 waves in wave order through LDS.
constexpr int AW_WAVES = 16, AW_DEPTH = 4;

template <int HD>
__global__ void __launch_bounds__(AW_WAVES * 64) attn_decode_wide_kernel(
    const bf16_t* __restrict__ qkv, bf16_t* __restrict__ kc, bf16_t* __restrict__ vc,
    const int32_t* __restrict__ pos_ptr, int Tmax, int H, int left, float scale,
    bf16_t* __restrict__ out) {
  constexpr int LPK = HD / 8, KPB = 64 / LPK;
  const int pos = *pos_ptr;
  __shared__ float wmax[AW_WAVES], wsum[AW_WAVES];
  __shared__ float wo[AW_WAVES][HD];
  const int bh = blockIdx.x, b = bh / H, h = bh - b * H;
  const int C = H * HD, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kk = lane / LPK, dp = lane % LPK;
  const bf16_t* row = qkv + (long)b * 3 * C;
  bf16_t* kb = kc + (long)bh * Tmax * HD;
  bf16_t* vb = vc + (long)bh * Tmax * HD;
  if (tid < LPK) {  // this position's key and value join the cache
    *(u32x4*)(kb + (long)pos * HD + tid * 8) = *(const u32x4*)(row + C + h * HD + tid * 8);
    *(u32x4*)(vb + (long)pos * HD + tid * 8) = *(const u32x4*)(row + 2 * C + h * HD + tid * 8);
  }
  const u32x4 qv = *(const u32x4*)(row + h * HD + dp * 8);
  const float q[8] = {bf_lo(qv.x) * scale, bf_hi(qv.x) * scale, bf_lo(qv.y) * scale,
                      bf_hi(qv.y) * scale, bf_lo(qv.z) * scale, bf_hi(qv.z) * scale,
                      bf_lo(qv.w) * scale, bf_hi(qv.w) * scale};
  const int j0 = left < 0 ? 0 : max(0, pos - left);
  float m = -FLT_MAX, l = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  constexpr int STRIDE = AW_WAVES * KPB;
  for (int jr = j0 + wave * KPB; jr <= pos; jr += AW_DEPTH * STRIDE) {
    u32x4 kv[AW_DEPTH], vv[AW_DEPTH];
#pragma unroll
    for (int i = 0; i < AW_DEPTH; ++i) {
      const int j = jr + i * STRIDE + kk;
      kv[i] = u32x4{0, 0, 0, 0};
      vv[i] = kv[i];
      if (j <= pos) {
        // the current position reads its own key / value from qkv (the cache
        // row is written above by other lanes; reading qkv avoids relying on it)
        const bf16_t* kr = j == pos ? row + C + h * HD : kb + (long)j * HD;
        const bf16_t* vr = j == pos ? row + 2 * C + h * HD : vb + (long)j * HD;
        kv[i] = *(const u32x4*)(kr + dp * 8);
        vv[i] = *(const u32x4*)(vr + dp * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < AW_DEPTH; ++i) {
      const int j = jr + i * STRIDE + kk;
      const u32x4 k = kv[i];
      float s = q[0] * bf_lo(k.x);
      s = fmaf(q[1], bf_hi(k.x), s);
      s = fmaf(q[2], bf_lo(k.y), s);
      s = fmaf(q[3], bf_hi(k.y), s);
      s = fmaf(q[4], bf_lo(k.z), s);
      s = fmaf(q[5], bf_hi(k.z), s);
      s = fmaf(q[6], bf_lo(k.w), s);
      s = fmaf(q[7], bf_hi(k.w), s);
#pragma unroll
      for (int off = LPK / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      if (j <= pos) {
        const u32x4 v = vv[i];
        const float vf[8] = {bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y),
                             bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w)};
        const float mn = fmaxf(m, s);
        const float corr = __expf(m - mn), p = __expf(s - mn);
        l = l * corr + p;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[d] = o[d] * corr + p * vf[d];
        m = mn;
      }
    }
  }
  // merge the key slots of the wave (lanes that differ in kk)
  float M = m;
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float f = l > 0.f ? __expf(m - M) : 0.f;
  float L = l * f;
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] *= f;
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    L += __shfl_xor(L, off);
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] += __shfl_xor(o[d], off);
  }
  if (kk == 0) {
#pragma unroll
    for (int d = 0; d < 8; ++d) wo[wave][dp * 8 + d] = o[d];
    if (dp == 0) {
      wmax[wave] = M;
      wsum[wave] = L;
    }
  }
  __syncthreads();
  if (tid < HD) {
    float Mx = -FLT_MAX;
#pragma unroll
    for (int w = 0; w < AW_WAVES; ++w) Mx = fmaxf(Mx, wmax[w]);
    float Ls = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < AW_WAVES; ++w) {
      const float g = wsum[w] > 0.f ? __expf(wmax[w] - Mx) : 0.f;
      Ls += wsum[w] * g;
      acc += wo[w][tid] * g;
    }
    out[(long)b * C + h * HD + tid] = f2bf(acc / Ls);
  }
}

// Few-row product of the decode step (bf16): out[b, n] = epilogue(sum_k
// a[b, k] W[n, k]) for the B rows (one per sequence) against a [N, K] weight,
// on MFMA 16x16x32: the first operand is 16 weight rows (output columns), the
// second 16 activation rows, so weight and activation loads go 1:1.
//
// Grid (column tiles of 16, row groups of 16); 4 waves per workgroup take
// interleaved 64-wide k blocks (lane quarter q holds k = 16q..16q+15 of a
// block, the same k for both operands, fed as two 8-deep halves), RL_DEPTH
// blocks of loads at a time with the next weights in flight behind the
// MFMAs, then sum in wave order through LDS and apply the epilogue.  All of K
// stays in one workgroup: a product is one launch with no partials to reduce.
// (Splitting k over workgroups with a last-arriver reduction measured several
// times slower: each writer's device-scope release writes back its XCD's L2.)
//
// With LNV > 0 the activation rows are LayerNorm(x) of the fp32 residual
// stream, computed by each workgroup into LDS first (one wave per row, all
// rows' loads issued together, the same arithmetic as the LayerNorm kernel, so
// the operand is bit-identical to the unfused one).
constexpr int RL_DEPTH = 4;

template <int WAVES>
__device__ __forceinline__ void rl_load(u32x4 (&v)[RL_DEPTH][2], const bf16_t* p, int kb0,
                                        int kend) {
#pragma unroll
  for (int i = 0; i < RL_DEPTH; ++i) {
    const int kb = kb0 + i * WAVES;  // wave-uniform
    if (kb < kend) {
      v[i][0] = *(const u32x4*)(p + kb * 64);
      v[i][1] = *(const u32x4*)(p + kb * 64 + 8);
    }
  }
}

template <int EPI, int WAVES, int LNV>
__global__ void __launch_bounds__(WAVES * 64) rows_linear_kernel(
    const bf16_t* __restrict__ a, const float* __restrict__ x, const float* __restrict__ lnw,
    const float* __restrict__ lnb, float eps, int B, int K, const bf16_t* __restrict__ W, int N,
    const float* __restrict__ bias, void* out, long ldo, const float* resid, bf16_t* aux,
    int tanh_form) {
  static_assert(WAVES >= 4 && (LNV == 0 || WAVES == 4), "256-thread epilogue, 4-row prologue");
  constexpr int STEP = RL_DEPTH * WAVES;
  __shared__ float part[WAVES * 64 * 4];
  extern __shared__ __align__(16) bf16_t xs[];  // LNV > 0: 16 rows, stride K + 8
  // The wave index in a scalar register: the block conditions below are then
  // scalar branches.  Derived per lane they compile to EXEC-masked regions,
  // and an MFMA in such a region still runs when EXEC is zero, accumulating
  // whatever its operand registers hold.
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16, b0 = blockIdx.y * 16;
  const int li = lane & 15, kq = lane >> 4;
  const int KB = K / 64, LDX = K + 8;  // K % 64 == 0
  // Rows past N (or B) read a valid row instead: MFMA output (n, b) depends
  // on weight row n and activation row b alone, and such outputs are dropped.
  const bf16_t* wrow = W + (long)min(n0 + li, N - 1) * K + kq * 16;
  u32x4 wv[RL_DEPTH][2], xv[RL_DEPTH][2];
  rl_load<WAVES>(wv, wrow, wave, KB);
  const bf16_t* xrow;
  if constexpr (LNV > 0) {
    constexpr int RPW = 16 / WAVES;
    const int C4 = K / 4;
    float4 v[RPW][LNV], g[LNV], be[LNV];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const float4* xr = (const float4*)(x + (long)min(b0 + wave + rr * WAVES, B - 1) * K);
#pragma unroll
      for (int i = 0; i < LNV; ++i) {
        const int c = lane + 64 * i;
        v[rr][i] = c < C4 ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int i = 0; i < LNV; ++i) {
      const int c = lane + 64 * i;
      g[i] = c < C4 ? ((const float4*)lnw)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      be[i] = lnb && c < C4 ? ((const float4*)lnb)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < LNV; ++i) s += (v[rr][i].x + v[rr][i].y) + (v[rr][i].z + v[rr][i].w);
      const float mu = warp_sum(s) / (float)K;
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < LNV; ++i) {
        if (lane + 64 * i < C4) {
          const float e0 = v[rr][i].x - mu, e1 = v[rr][i].y - mu, e2 = v[rr][i].z - mu,
                      e3 = v[rr][i].w - mu;
          q += (e0 * e0 + e1 * e1) + (e2 * e2 + e3 * e3);
        }
      }
      const float rs = 1.f / sqrtf(warp_sum(q) / (float)K + eps);
      const int r = wave + rr * WAVES;
#pragma unroll
      for (int i = 0; i < LNV; ++i) {
        const int c = lane + 64 * i;
        if (c < C4)
          *(uint2*)(xs + r * LDX + 4 * c) =
              make_uint2(pack_bf2((v[rr][i].x - mu) * rs * g[i].x + be[i].x,
                                  (v[rr][i].y - mu) * rs * g[i].y + be[i].y),
                         pack_bf2((v[rr][i].z - mu) * rs * g[i].z + be[i].z,
                                  (v[rr][i].w - mu) * rs * g[i].w + be[i].w));
      }
    }
    __syncthreads();
    xrow = xs + li * LDX + kq * 16;
  } else {
    xrow = a + (long)min(b0 + li, B - 1) * K + kq * 16;
  }
  rl_load<WAVES>(xv, xrow, wave, KB);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb0 = wave; kb0 < KB; kb0 += STEP) {
#pragma unroll
    for (int i = 0; i < RL_DEPTH; ++i) {
      if (kb0 + i * WAVES < KB) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wv[i][0]),
                                                      __builtin_bit_cast(bf16x8, xv[i][0]), acc,
                                                      0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wv[i][1]),
                                                      __builtin_bit_cast(bf16x8, xv[i][1]), acc,
                                                      0, 0, 0);
      }
    }
    rl_load<WAVES>(wv, wrow, kb0 + STEP, KB);  // both operands of the next batch
    rl_load<WAVES>(xv, xrow, kb0 + STEP, KB);
  }
  // acc item r of lane l: output column n0 + 4 (l / 16) + r, row b0 + l % 16.
  *(f32x4*)(part + (wave * 64 + lane) * 4) = acc;
  __syncthreads();
  const int t = threadIdx.x, l = t >> 2, r = t & 3;  // one (column, row) per thread
  if (t >= 256) return;
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) v += part[(w * 64 + l) * 4 + r];
  const int n = n0 + 4 * (l >> 4) + r, b = b0 + (l & 15);
  if (n < N && b < B) {
    if (bias) v += bias[n];
    const long o = (long)b * ldo + n;
    if constexpr (EPI == GPT_EPI_RESIDUAL) {
      ((float*)out)[o] = resid[o] + v;
    } else {
      const bf16_t u = f2bf(v);
      ((bf16_t*)out)[o] = u;
      if constexpr (EPI == GPT_EPI_GELU) {  // GELU of the stored (rounded) pre-activation
        if (aux) aux[o] = f2bf(gelu_fast(bf2f(u), tanh_form));
      }
    }
  }
}

constexpr int SK_THREADS = 1024;

__device__ __forceinline__ uint32_t order_key(float f) {  // larger float -> larger key
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename ActT>
__global__ void __launch_bounds__(SK_THREADS) sample_kernel(
    const ActT* __restrict__ z, long ldz, int V, float temperature, int top_k,
    const float* __restrict__ u, long u_stride, int32_t* __restrict__ tok,
    int32_t* __restrict__ seq, long seq_stride, int seq_col) {
  __shared__ uint32_t hist[256];
  __shared__ float fv[SK_THREADS];
  __shared__ int iv[SK_THREADS];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_krem, s_pick;
  const int b = blockIdx.x, tid = threadIdx.x;
  const ActT* row = z + (long)b * ldz;
  int result = 0;
  if (temperature == 0.f) {
    // argmax, the lowest index among equal maxima
    float best = -FLT_MAX;
    int bi = V;
    for (int i = tid; i < V; i += SK_THREADS) {
      const float v = Act<ActT>::load(row, i);
      if (v > best) { best = v; bi = i; }
    }
    fv[tid] = best;
    iv[tid] = bi;
    __syncthreads();
    for (int w = SK_THREADS / 2; w > 0; w >>= 1) {
      if (tid < w) {
        const float a = fv[tid], c = fv[tid + w];
        const int ia = iv[tid], ic = iv[tid + w];
        if (c > a || (c == a && ic < ia)) { fv[tid] = c; iv[tid] = ic; }
      }
      __syncthreads();
    }
    result = iv[0];
  } else {
    // threshold key of the top_k-th largest w = z / temperature (0: keep all)
    uint32_t thr = 0;
    if (top_k > 0 && top_k < V) {
      uint32_t prefix = 0, mask = 0;
      int krem = top_k;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < V; i += SK_THREADS) {
          const uint32_t k = order_key(__fdiv_rn(Act<ActT>::load(row, i), temperature));
          if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1u);
        }
        __syncthreads();
        if (tid == 0) {
          int acc = 0, d = 255;
          for (; d > 0; --d) {
            if (acc + (int)hist[d] >= krem) break;
            acc += (int)hist[d];
          }
          s_krem = krem - acc;
          s_prefix = prefix | ((uint32_t)d << shift);
          s_mask = mask | (255u << shift);
        }
        __syncthreads();
        prefix = s_prefix;
        mask = s_mask;
        krem = s_krem;
        __syncthreads();
      }
      thr = prefix;
    }
    // maximum of the kept values
    float mx = -FLT_MAX;
    for (int i = tid; i < V; i += SK_THREADS) {
      const float w = __fdiv_rn(Act<ActT>::load(row, i), temperature);
      if (order_key(w) >= thr) mx = fmaxf(mx, w);
    }
    fv[tid] = mx;
    __syncthreads();
    for (int w = SK_THREADS / 2; w > 0; w >>= 1) {
      if (tid < w) fv[tid] = fmaxf(fv[tid], fv[tid + w]);
      __syncthreads();
    }
    const float M = fv[0];
    __syncthreads();
    // per-thread sums over a contiguous chunk, then an exclusive scan in thread order
    const int ch = (V + SK_THREADS - 1) / SK_THREADS;
    const int i0 = min(V, tid * ch), i1 = min(V, i0 + ch);
    float sum = 0.f;
    int last_kept = -1;
    for (int i = i0; i < i1; ++i) {
      const float w = __fdiv_rn(Act<ActT>::load(row, i), temperature);
      if (order_key(w) >= thr) {
        sum += __expf(w - M);
        last_kept = i;
      }
    }
    fv[tid] = sum;
    iv[tid] = last_kept;
    if (tid == 0) s_pick = SK_THREADS;
    __syncthreads();
    // Hillis-Steele inclusive scan (a fixed sequence of additions)
    for (int w = 1; w < SK_THREADS; w <<= 1) {
      const float add = tid >= w ? fv[tid - w] : 0.f;
      __syncthreads();
      fv[tid] += add;
      __syncthreads();
    }
    const float incl = fv[tid], excl = incl - sum;  // excl: this thread's start
    const float total = fv[SK_THREADS - 1];
    const float target = u[(long)b * u_stride] * total;
    if (sum > 0.f && excl <= target && target < incl) atomicMin(&s_pick, tid);
    // the last thread with kept entries is the fallback when rounding leaves target >= total
    __syncthreads();
    for (int w = SK_THREADS / 2; w > 0; w >>= 1) {
      if (tid < w) iv[tid] = max(iv[tid], iv[tid + w]);
      __syncthreads();
    }
    const int fallback = iv[0];
    const int pick = s_pick;
    __syncthreads();  // every thread has read s_pick before it is reused below
    if (pick == SK_THREADS) {
      result = fallback;
    } else {
      if (tid == pick) {
        float acc = excl;
        int r = last_kept;
        for (int i = i0; i < i1; ++i) {
          const float w = __fdiv_rn(Act<ActT>::load(row, i), temperature);
          if (order_key(w) >= thr) {
            acc += __expf(w - M);
            if (acc > target) { r = i; break; }
          }
        }
        s_pick = r;  // reuse: the chosen index
      }
      __syncthreads();
      result = s_pick;
    }
  }
  if (tid == 0) {
    tok[b] = result;
    if (seq) seq[(long)b * seq_stride + seq_col] = result;
  }
}

__global__ void gather_column_kernel(const int32_t* __restrict__ seq, long stride, int col, int B,
                                     int32_t* __restrict__ tok) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) tok[b] = seq[(long)b * stride + col];
}

__global__ void copy_prompt_kernel(const int32_t* __restrict__ prompt, int T0, int Ltot, int B,
                                   int32_t* __restrict__ out) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (long)B * T0) {
    const long b = i / T0, t = i - b * T0;
    out[b * Ltot + t] = prompt[i];
  }
}

// The decode position lives in device memory, so a captured step serves
// every position: set at a reset, advanced by the last kernel of a step.
__global__ void gen_set_pos_kernel(int32_t* pos, int32_t v) {
  if (threadIdx.x == 0) *pos = v;
}
__global__ void gen_advance_kernel(int32_t* pos) {
  if (threadIdx.x == 0) *pos += 1;
}

}  // namespace

hipError_t gen_embed(const int32_t* tok, const float* wte, const float* wpe, const int32_t* pos,
                     int B, int C, int V, float* x, hipStream_t s) {
  gen_embed_kernel<<<B, 256, 0, s>>>(tok, wte, wpe, pos, C, V, x);
  return hipGetLastError();
}

hipError_t gen_set_pos(int32_t* pos, int32_t v, hipStream_t s) {
  gen_set_pos_kernel<<<1, 64, 0, s>>>(pos, v);
  return hipGetLastError();
}

hipError_t gen_advance(int32_t* pos, hipStream_t s) {
  gen_advance_kernel<<<1, 64, 0, s>>>(pos);
  return hipGetLastError();
}

template <int EPI, int WAVES, int LNV>
hipError_t rows_linear_go(const RowsLinear& p, hipStream_t s) {
  const dim3 grid((unsigned)((p.N + 15) / 16), (unsigned)((p.B + 15) / 16));
  const size_t lds = LNV > 0 ? (size_t)16 * (p.K + 8) * sizeof(bf16_t) : 0;
  rows_linear_kernel<EPI, WAVES, LNV><<<grid, WAVES * 64, lds, s>>>(
      (const bf16_t*)p.a, p.x, p.ln_w, p.ln_b, p.eps, p.B, p.K, (const bf16_t*)p.W, p.N, p.bias,
      p.out, p.ldo, p.resid, (bf16_t*)p.aux, p.tanh_form);
  return hipGetLastError();
}

template <int EPI>
hipError_t rows_linear_epi(const RowsLinear& p, hipStream_t s) {
  if constexpr (EPI != GPT_EPI_RESIDUAL) {
    if (p.x) {  // LayerNorm prologue: one float4 per lane per 256 columns
      const int nv = (p.K / 4 + 63) / 64;
      if (nv <= 1) return rows_linear_go<EPI, 4, 1>(p, s);
      if (nv <= 2) return rows_linear_go<EPI, 4, 2>(p, s);
      if (nv <= 3) return rows_linear_go<EPI, 4, 3>(p, s);
      return rows_linear_go<EPI, 4, 4>(p, s);  // K <= 1024
    }
  }
  // 16 waves when 4 would need more than one batch of loads per wave
  if (p.K / 64 > 4 * RL_DEPTH) return rows_linear_go<EPI, 16, 0>(p, s);
  return rows_linear_go<EPI, 4, 0>(p, s);
}

hipError_t rows_linear(const RowsLinear& p, hipStream_t s) {
  if (p.B <= 0 || p.N <= 0) return hipSuccess;
  if (p.K % 64 || (!p.a && !p.x) || (p.x && (!p.ln_w || p.K > ROWS_LINEAR_MAX_LN_K)) ||
      (p.B + 15) / 16 > 65535)
    return hipErrorInvalidValue;
  if (p.epi == GPT_EPI_STORE) return rows_linear_epi<GPT_EPI_STORE>(p, s);
  if (p.epi == GPT_EPI_GELU) return rows_linear_epi<GPT_EPI_GELU>(p, s);
  if (p.epi == GPT_EPI_RESIDUAL && !p.x) return rows_linear_epi<GPT_EPI_RESIDUAL>(p, s);
  return hipErrorInvalidValue;
}

bool attn_decode_supported(int hd) { return hd == 32 || hd == 64 || hd == 128; }

hipError_t attn_decode(int prec, int hd, const void* qkv, void* kc, void* vc, const int32_t* pos,
                       int Tmax, int B, int H, int left, void* out, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)hd);
#define AD_(T, D)                                                                            \
  attn_decode_kernel<T, D><<<B * H, AD_THREADS, 0, s>>>((const T*)qkv, (T*)kc, (T*)vc, pos, \
                                                        Tmax, H, left, scale, (T*)out)
#define AW_(D)                                                                           \
  attn_decode_wide_kernel<D><<<B * H, AW_WAVES * 64, 0, s>>>(                          \
      (const bf16_t*)qkv, (bf16_t*)kc, (bf16_t*)vc, pos, Tmax, H, left, scale, (bf16_t*)out)
  if (prec == GPT_BF16) {
    if (hd == 32) AW_(32);
    else if (hd == 64) AW_(64);
    else if (hd == 128) AW_(128);
    else return hipErrorInvalidValue;
  } else {
    if (hd == 32) AD_(float, 32);
    else if (hd == 64) AD_(float, 64);
    else if (hd == 128) AD_(float, 128);
    else return hipErrorInvalidValue;
  }
#undef AD_
#undef AW_
  return hipGetLastError();
}

hipError_t sample(int prec, const void* logits, long ldz, int B, int V, float temperature,
                  int top_k, const float* u, long u_stride, int32_t* tok, int32_t* seq,
                  long seq_stride, int seq_col, hipStream_t s) {
  if (prec == GPT_BF16)
    sample_kernel<bf16_t><<<B, SK_THREADS, 0, s>>>((const bf16_t*)logits, ldz, V, temperature,
                                                   top_k, u, u_stride, tok, seq, seq_stride,
                                                   seq_col);
  else
    sample_kernel<float><<<B, SK_THREADS, 0, s>>>((const float*)logits, ldz, V, temperature, top_k,
                                                  u, u_stride, tok, seq, seq_stride, seq_col);
  return hipGetLastError();
}

hipError_t gather_column(const int32_t* seq, long stride, int col, int B, int32_t* tok,
                         hipStream_t s) {
  gather_column_kernel<<<(B + 255) / 256, 256, 0, s>>>(seq, stride, col, B, tok);
  return hipGetLastError();
}

hipError_t copy_prompt(const int32_t* prompt, int T0, int Ltot, int B, int32_t* out,
                       hipStream_t s) {
  const long n = (long)B * T0;
  if (n == 0) return hipSuccess;
  copy_prompt_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(prompt, T0, Ltot, B, out);
  return hipGetLastError();
}

}  // namespace gpt
