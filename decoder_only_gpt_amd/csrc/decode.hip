// Generation with a key/value cache: the kernels of one decode step that the
// training step does not have (nanoGPT README, "sampling / inference":
// sample.py continues a prompt token by token; llm.c summary, "Sampling").
//
//   gen_embed      x[b] = wte[token[b]] + wpe[pos]
//   attn_decode    one query per (sequence, head) against the cached keys and
//                  values 0..pos-1 plus its own (written to the cache here);
//                  each thread takes every 256th key with a running softmax,
//                  the block combines in a fixed order
//   sample         temperature / top-k / inverse-CDF draw per sequence (one
//                  1024-thread block per row): the top-k threshold by a 4-pass
//                  radix select on order-preserving keys, the cumulative sum by
//                  a fixed-order scan of per-thread chunks, so the same logits
//                  and u always give the same token
// The matrix products and LayerNorms of the step are the training kernels
// run on B rows.

#include "common.h"
#include "kernels.h"

#include <cfloat>

namespace gpt {

namespace {

__global__ void __launch_bounds__(256) gen_embed_kernel(const int32_t* __restrict__ tok,
                                                        const float* __restrict__ wte,
                                                        const float* __restrict__ wpe, int pos,
                                                        int C, float* __restrict__ x) {
  const int b = blockIdx.x;
  const long t = tok[b];
  for (int c = threadIdx.x * 4; c < C; c += 256 * 4) {  // C % 64 == 0
    const float4 e = *(const float4*)(wte + t * C + c);
    const float4 p = *(const float4*)(wpe + (long)pos * C + c);
    *(float4*)(x + (long)b * C + c) = make_float4(e.x + p.x, e.y + p.y, e.z + p.z, e.w + p.w);
  }
}

constexpr int AD_THREADS = 256;

template <typename ActT, int HD>
__global__ void __launch_bounds__(AD_THREADS) attn_decode_kernel(
    const ActT* __restrict__ qkv, ActT* __restrict__ kc, ActT* __restrict__ vc, int pos,
    int Tmax, int H, int left, float scale, ActT* __restrict__ out) {
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

}  // namespace

hipError_t gen_embed(const int32_t* tok, const float* wte, const float* wpe, int pos, int B, int C,
                     float* x, hipStream_t s) {
  gen_embed_kernel<<<B, 256, 0, s>>>(tok, wte, wpe, pos, C, x);
  return hipGetLastError();
}

bool attn_decode_supported(int hd) { return hd == 32 || hd == 64 || hd == 128; }

hipError_t attn_decode(int prec, int hd, const void* qkv, void* kc, void* vc, int pos, int Tmax,
                       int B, int H, int left, void* out, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)hd);
#define AD_(T, D)                                                                            \
  attn_decode_kernel<T, D><<<B * H, AD_THREADS, 0, s>>>((const T*)qkv, (T*)kc, (T*)vc, pos, \
                                                        Tmax, H, left, scale, (T*)out)
  if (prec == GPT_BF16) {
    if (hd == 32) AD_(bf16_t, 32);
    else if (hd == 64) AD_(bf16_t, 64);
    else if (hd == 128) AD_(bf16_t, 128);
    else return hipErrorInvalidValue;
  } else {
    if (hd == 32) AD_(float, 32);
    else if (hd == 64) AD_(float, 64);
    else if (hd == 128) AD_(float, 128);
    else return hipErrorInvalidValue;
  }
#undef AD_
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
