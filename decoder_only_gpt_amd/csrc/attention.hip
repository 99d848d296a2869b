// Causal multi-head self-attention with an optional left window, forward and
// backward.
//
// What is computed (nanoGPT README: "6-layer Transformer with 6 heads";
// nanochat "FLOPs-Berechnung im Detail": per-layer (left, right) window, the
// effective sequence is min(window, T)): for each batch row and head,
// S = q k^T / sqrt(hd), key j visible to query i iff i - left <= j <= i
// (left < 0: j <= i), P = softmax_j(S), y = P v.  The log-sum-exp of each
// query's scores is kept so the backward can rebuild P exactly (the llm.c
// summary, "Configuración mínima del entorno", names cuDNN FlashAttention for
// this step; the tiled online-softmax scheme below is written for CDNA4).
//
// bf16 path (head_dim 32/64/128), CDNA4 MFMA 32x32x16:
//   forward: a workgroup owns 128 queries of one (batch, head), one wave per
//   32 queries.  Each wave computes S^T = K Q^T for 64-key blocks, so every
//   lane owns ONE query column: the running max / sum are per-lane scalars and
//   a row reduction is one cross-half swap.  P^T stays in registers and feeds
//   O^T += V^T P^T directly.  K and V tiles sit in LDS in their natural layout;
//   operands that need the transposed view are fetched with the LDS transpose
//   read.  Blocks entirely outside a wave's causal band / window are skipped.
//   backward: two deterministic kernels (no atomics).  dK/dV: a wave owns 32
//   keys and walks the query blocks that can see them.  dQ: a wave owns 32
//   queries and walks their key blocks.  Both rebuild P from the saved LSE.
// fp32 path: one wave per (query) or (key) row with exact fp32 arithmetic.

#include "common.h"
#include "kernels.h"

namespace gpt {

namespace {

constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ bool visible(int i, int j, int left, int T) {
  return j <= i && j < T && (left < 0 || i - j <= left);
}

// ---------------------------------------------------------------------------
// fp32 (generic-type) kernels: one wave per row, lanes split the head dim.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) attn_fwd_rows(const T* qkv, T* out, float* lse, int B,
                                                     int Tn, int H, int hd, int left, float scale) {
  const int lane = threadIdx.x & 63;
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (long)B * H * Tn) return;
  const int i = (int)(w % Tn);
  const int h = (int)((w / Tn) % H);
  const int b = (int)(w / ((long)Tn * H));
  const long C = (long)H * hd, ld = 3 * C;
  const T* q = qkv + (long)(b * Tn + i) * ld + h * hd;
  float q0 = lane < hd ? Act<T>::load(q, lane) : 0.f;
  float q1 = lane + 64 < hd ? Act<T>::load(q, lane + 64) : 0.f;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  const int j0 = left < 0 ? 0 : max(0, i - left);
  for (int j = j0; j <= i; ++j) {
    const T* k = qkv + (long)(b * Tn + j) * ld + C + h * hd;
    const T* v = k + C;
    float k0 = lane < hd ? Act<T>::load(k, lane) : 0.f;
    float k1 = lane + 64 < hd ? Act<T>::load(k, lane + 64) : 0.f;
    float s = warp_sum(q0 * k0 + q1 * k1) * scale;
    float mn = fmaxf(m, s);
    float alpha = expf(m - mn), p = expf(s - mn);
    float v0 = lane < hd ? Act<T>::load(v, lane) : 0.f;
    float v1 = lane + 64 < hd ? Act<T>::load(v, lane + 64) : 0.f;
    l = l * alpha + p;
    o0 = o0 * alpha + p * v0;
    o1 = o1 * alpha + p * v1;
    m = mn;
  }
  T* o = out + (long)(b * Tn + i) * C + h * hd;
  if (lane < hd) Act<T>::store(o, lane, o0 / l);
  if (lane + 64 < hd) Act<T>::store(o, lane + 64, o1 / l);
  if (lane == 0) lse[((long)b * H + h) * Tn + i] = m + logf(l);
}

// D[b,h,i] = sum_d dO[i,d] * O[i,d]  (one thread per (row, head)).
// bf16: one wave per token row; a lane takes 8 consecutive head dims (16-byte
// loads) and the hd/8 lanes of a head combine by butterfly shuffles.
template <int HD>
__global__ void __launch_bounds__(256) attn_dvec_bf16(const bf16_t* out, const bf16_t* dout,
                                                      float* D, int M, int Tn, int H) {
  constexpr int LPH = HD / 8;  // lanes per head
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int C = H * HD;
  const int b = (int)(row / Tn), t = (int)(row % Tn);
  for (int v0 = 0; v0 < C / 8; v0 += 64) {
    const int v = v0 + lane;
    float s = 0.f;
    if (v < C / 8) {
      u32x4 a = *(const u32x4*)(out + row * C + v * 8);
      u32x4 g = *(const u32x4*)(dout + row * C + v * 8);
#pragma unroll
      for (int k = 0; k < 4; ++k) s += bf_lo(a[k]) * bf_lo(g[k]) + bf_hi(a[k]) * bf_hi(g[k]);
    }
#pragma unroll
    for (int o = 1; o < LPH; o <<= 1) s += __shfl_xor(s, o, 64);
    if (v < C / 8 && (lane % LPH) == 0) {
      const int h = v / LPH;
      D[((long)b * H + h) * Tn + t] = s;
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(256) attn_dvec(const T* out, const T* dout, float* D, int B,
                                                 int Tn, int H, int hd) {
  long t = (long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long)B * Tn * H) return;
  int h = (int)(t % H);
  long row = t / H;
  int i = (int)(row % Tn), b = (int)(row / Tn);
  const long C = (long)H * hd;
  const T* o = out + row * C + h * hd;
  const T* d = dout + row * C + h * hd;
  float s = 0.f;
  for (int e = 0; e < hd; ++e) s += Act<T>::load(o, e) * Act<T>::load(d, e);
  D[((long)b * H + h) * Tn + i] = s;
}

template <typename T>
__global__ void __launch_bounds__(256) attn_dq_rows(const T* qkv, const float* lse, const T* dout,
                                                    const float* D, T* dqkv, int B, int Tn, int H,
                                                    int hd, int left, float scale) {
  const int lane = threadIdx.x & 63;
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (long)B * H * Tn) return;
  const int i = (int)(w % Tn);
  const int h = (int)((w / Tn) % H);
  const int b = (int)(w / ((long)Tn * H));
  const long C = (long)H * hd, ld = 3 * C;
  const T* q = qkv + (long)(b * Tn + i) * ld + h * hd;
  const T* dO = dout + (long)(b * Tn + i) * C + h * hd;
  float q0 = lane < hd ? Act<T>::load(q, lane) : 0.f;
  float q1 = lane + 64 < hd ? Act<T>::load(q, lane + 64) : 0.f;
  float g0 = lane < hd ? Act<T>::load(dO, lane) : 0.f;
  float g1 = lane + 64 < hd ? Act<T>::load(dO, lane + 64) : 0.f;
  const long r = ((long)b * H + h) * Tn + i;
  const float L = lse[r], Di = D[r];
  float a0 = 0.f, a1 = 0.f;
  const int j0 = left < 0 ? 0 : max(0, i - left);
  for (int j = j0; j <= i; ++j) {
    const T* k = qkv + (long)(b * Tn + j) * ld + C + h * hd;
    const T* v = k + C;
    float k0 = lane < hd ? Act<T>::load(k, lane) : 0.f;
    float k1 = lane + 64 < hd ? Act<T>::load(k, lane + 64) : 0.f;
    float v0 = lane < hd ? Act<T>::load(v, lane) : 0.f;
    float v1 = lane + 64 < hd ? Act<T>::load(v, lane + 64) : 0.f;
    float s = warp_sum(q0 * k0 + q1 * k1) * scale;
    float dp = warp_sum(g0 * v0 + g1 * v1);
    float p = expf(s - L);
    float ds = p * (dp - Di);
    a0 += ds * k0;
    a1 += ds * k1;
  }
  T* dq = dqkv + (long)(b * Tn + i) * ld + h * hd;
  if (lane < hd) Act<T>::store(dq, lane, a0 * scale);
  if (lane + 64 < hd) Act<T>::store(dq, lane + 64, a1 * scale);
}

template <typename T>
__global__ void __launch_bounds__(256) attn_dkv_rows(const T* qkv, const float* lse,
                                                     const T* dout, const float* D, T* dqkv, int B,
                                                     int Tn, int H, int hd, int left,
                                                     float scale) {
  const int lane = threadIdx.x & 63;
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (long)B * H * Tn) return;
  const int j = (int)(w % Tn);
  const int h = (int)((w / Tn) % H);
  const int b = (int)(w / ((long)Tn * H));
  const long C = (long)H * hd, ld = 3 * C;
  const T* k = qkv + (long)(b * Tn + j) * ld + C + h * hd;
  const T* v = k + C;
  float k0 = lane < hd ? Act<T>::load(k, lane) : 0.f;
  float k1 = lane + 64 < hd ? Act<T>::load(k, lane + 64) : 0.f;
  float v0 = lane < hd ? Act<T>::load(v, lane) : 0.f;
  float v1 = lane + 64 < hd ? Act<T>::load(v, lane + 64) : 0.f;
  float dk0 = 0.f, dk1 = 0.f, dv0 = 0.f, dv1 = 0.f;
  const int i1 = left < 0 ? Tn - 1 : min(Tn - 1, j + left);
  for (int i = j; i <= i1; ++i) {
    const T* q = qkv + (long)(b * Tn + i) * ld + h * hd;
    const T* dO = dout + (long)(b * Tn + i) * C + h * hd;
    float q0 = lane < hd ? Act<T>::load(q, lane) : 0.f;
    float q1 = lane + 64 < hd ? Act<T>::load(q, lane + 64) : 0.f;
    float g0 = lane < hd ? Act<T>::load(dO, lane) : 0.f;
    float g1 = lane + 64 < hd ? Act<T>::load(dO, lane + 64) : 0.f;
    const long r = ((long)b * H + h) * Tn + i;
    float s = warp_sum(q0 * k0 + q1 * k1) * scale;
    float dp = warp_sum(g0 * v0 + g1 * v1);
    float p = expf(s - lse[r]);
    float ds = p * (dp - D[r]);
    dv0 += p * g0;
    dv1 += p * g1;
    dk0 += ds * q0;
    dk1 += ds * q1;
  }
  T* dk = dqkv + (long)(b * Tn + j) * ld + C + h * hd;
  T* dv = dk + C;
  if (lane < hd) {
    Act<T>::store(dk, lane, dk0 * scale);
    Act<T>::store(dv, lane, dv0);
  }
  if (lane + 64 < hd) {
    Act<T>::store(dk, lane + 64, dk1 * scale);
    Act<T>::store(dv, lane + 64, dv1);
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernels.
// ---------------------------------------------------------------------------
constexpr int KB = 64;  // keys (forward / dQ) or queries (dK/dV) per LDS block

// LDS row pitch of a [64][HD] tile: HD + 24 bf16 puts any 16 consecutive rows
// of a 16-byte fragment read on distinct 4-bank groups and the four rows of a
// transpose read (32 bytes each) on disjoint banks, for 64 (or 32) banks.
template <int HD> constexpr int pitch_of() { return HD + 24; }

// Rows [row0, row0+64) x HD of a strided bf16 matrix into LDS [64][pitch];
// rows >= nrows read as zero.
template <int HD>
__device__ __forceinline__ void lds_rows(const bf16_t* src, long ld, int row0, int nrows,
                                         bf16_t* dst) {
  constexpr int VPR = HD / 8, P = pitch_of<HD>();  // 16-byte vectors per row
  for (int u = threadIdx.x; u < KB * VPR; u += 256) {
    int r = u / VPR, c = (u % VPR) * 8;
    u32x4 val = {0, 0, 0, 0};
    if (row0 + r < nrows) val = *(const u32x4*)(src + (long)(row0 + r) * ld + c);
    *(u32x4*)(dst + r * P + c) = val;
  }
}

// Register staging of one [64][HD] tile: vector v = t + 256 i covers row
// v / (HD/8), head dims (v % (HD/8)) * 8 .. + 7.  Loading the next block into
// registers while the current one is multiplied hides the global latency.
template <int HD> struct TileRegs { u32x4 v[(KB * HD / 8 + 255) / 256]; };

template <int HD>
__device__ __forceinline__ void tile_load(const bf16_t* src, long ld, int row0, int nrows,
                                          TileRegs<HD>& t) {
  constexpr int VPR = HD / 8, NV = (KB * HD / 8 + 255) / 256;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int u = threadIdx.x + 256 * i;
    const int r = u / VPR, c = (u % VPR) * 8;
    u32x4 val = {0, 0, 0, 0};
    if (u < KB * VPR && row0 + r < nrows) val = *(const u32x4*)(src + (long)(row0 + r) * ld + c);
    t.v[i] = val;
  }
}

template <int HD>
__device__ __forceinline__ void tile_store(const TileRegs<HD>& t, bf16_t* dst) {
  constexpr int VPR = HD / 8, NV = (KB * HD / 8 + 255) / 256, P = pitch_of<HD>();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int u = threadIdx.x + 256 * i;
    if (u < KB * VPR) *(u32x4*)(dst + (u / VPR) * P + (u % VPR) * 8) = t.v[i];
  }
}

// MFMA operand fragment whose lane index (lane % 32) runs along the row of a
// tile: row r0 + lane % 32, head dims 16 st + 8 (lane / 32) + 0..7.
template <int HD>
__device__ __forceinline__ bf16x8 row_frag(const bf16_t* t, int r0, int st, int lane) {
  return *(const bf16x8*)(t + (r0 + (lane & 31)) * pitch_of<HD>() + 16 * st + 8 * (lane >> 5));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// MFMA operand fragment whose lane index runs along the COLUMNS of a tile
// (head dim c0 + lane % 32) and whose 8 k-slots are tile rows in the order of
// a 32x32 accumulator handed on as an operand: rows base + 4 g + 0..3 and
// base + 8 + 4 g + 0..3, g = lane / 32.  Two LDS transpose reads: within each
// group of 16 lanes, source lane s = a + 4 b supplies (row kb + b, columns
// 4 a .. 4 a + 3) and lane j receives column j of rows kb .. kb + 3.
template <int HD>
__device__ __forceinline__ bf16x8 tr_slots(const bf16_t* t, int c0, int base, int lane) {
  constexpr int P = pitch_of<HD>();
  const int s = lane & 15, grp = lane >> 4;
  const int col = c0 + 16 * (grp & 1) + 4 * (s & 3);
  const int row = base + 4 * (grp >> 1) + (s >> 2);
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + row * P + col));
  v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + (row + 8) * P + col));
  v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return *(bf16x8*)&v;
}

// 8 accumulator values r = 8*s2 .. 8*s2+7 of a 32x32 block as a bf16 operand.
__device__ __forceinline__ bf16x8 acc_slots(const f32x16& acc, int s2) {
  u32x4 v{pack_bf2(acc[8 * s2 + 0], acc[8 * s2 + 1]), pack_bf2(acc[8 * s2 + 2], acc[8 * s2 + 3]),
          pack_bf2(acc[8 * s2 + 4], acc[8 * s2 + 5]), pack_bf2(acc[8 * s2 + 6], acc[8 * s2 + 7])};
  return *(bf16x8*)&v;
}

__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

template <int HD>
__global__ void __launch_bounds__(256) attn_fwd_mfma(const bf16_t* qkv, bf16_t* out, float* lse,
                                                     int Tn, int H, int left, float scale_log2) {
  constexpr int P = pitch_of<HD>(), NS = HD / 16, ND = HD / 32;
  __shared__ __attribute__((aligned(16))) bf16_t Kbuf[2][KB * P];
  __shared__ __attribute__((aligned(16))) bf16_t Vbuf[2][KB * P];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int h = blockIdx.y, b = blockIdx.z;
  const long C = (long)H * HD, ld = 3 * C;
  const bf16_t* base = qkv + (long)b * Tn * ld;
  const int qblk0 = blockIdx.x * 128;
  const int qw0 = qblk0 + wave * 32;
  const int qi = qw0 + c;  // this lane's query

  bf16x8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4 v{0, 0, 0, 0};
    if (qi < Tn) v = *(const u32x4*)(base + (long)qi * ld + h * HD + 16 * s + 8 * g);
    qf[s] = *(bf16x8*)&v;
  }
  f32x16 o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  float mrow = -1e30f, lrow = 0.f;

  const int qlast = min(Tn - 1, qblk0 + 127);
  const int kfirst = left < 0 ? 0 : max(0, qblk0 - left);
  const int kstart = (kfirst / KB) * KB;
  TileRegs<HD> rk, rv;
  tile_load<HD>(base + C + h * HD, ld, kstart, Tn, rk);
  tile_load<HD>(base + 2 * C + h * HD, ld, kstart, Tn, rv);
  tile_store<HD>(rk, Kbuf[0]);
  tile_store<HD>(rv, Vbuf[0]);
  __syncthreads();
  int buf = 0;
  for (int kb0 = kstart; kb0 <= qlast; kb0 += KB, buf ^= 1) {
    const bf16_t* Ks = Kbuf[buf];
    const bf16_t* Vs = Vbuf[buf];
    const bool more = kb0 + KB <= qlast;
    if (more) {  // next block's tiles travel while this one is multiplied
      tile_load<HD>(base + C + h * HD, ld, kb0 + KB, Tn, rk);
      tile_load<HD>(base + 2 * C + h * HD, ld, kb0 + KB, Tn, rv);
    }
    const bool skip = kb0 > qw0 + 31 || (left >= 0 && kb0 + KB - 1 < qw0 - left);
    if (!skip) {
    // every (query, key) of this wave and block visible: no per-element mask
    const bool full = kb0 + KB - 1 <= qw0 && qw0 + 31 < Tn && (left < 0 || qw0 + 31 - kb0 <= left);
    f32x16 s[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kk][r] = 0.f;
#pragma unroll
      for (int st = 0; st < NS; ++st)
        s[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<HD>(Ks, kk * 32, st, lane), qf[st],
                                                        s[kk], 0, 0, 0);
    }
    // s[kk][r]: key kb0 + kk*32 + acc_row(r, g), query qi (scaled to log2 units below)
    float mx = -1e30f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int j = kb0 + kk * 32 + acc_row(r, g);
        float v = (full || visible(qi, j, left, Tn)) ? s[kk][r] * scale_log2 : -INFINITY;
        s[kk][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(mrow, mx);
    const float alpha = exp2f(mrow - mnew);
    float ls = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = exp2f(s[kk][r] - mnew);
        s[kk][r] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 32, 64);
    lrow = lrow * alpha + ls;
    mrow = mnew;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
    // O^T[d][q] += V^T[d][key] P[key][q]
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 pf = acc_slots(s[kk], s2);
#pragma unroll
        for (int d = 0; d < ND; ++d)
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tr_slots<HD>(Vs, d * 32, kk * 32 + 16 * s2, lane), pf, o[d], 0, 0, 0);
      }
    }  // !skip
    if (more) {
      tile_store<HD>(rk, Kbuf[buf ^ 1]);
      tile_store<HD>(rv, Vbuf[buf ^ 1]);
    }
    __syncthreads();
  }
  if (qi < Tn) {
    const float inv = 1.f / lrow;
    bf16_t* orow = out + ((long)b * Tn + qi) * C + h * HD;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        int dd = d * 32 + 8 * r4 + 4 * g;
        uint2 w = make_uint2(pack_bf2(o[d][4 * r4 + 0] * inv, o[d][4 * r4 + 1] * inv),
                             pack_bf2(o[d][4 * r4 + 2] * inv, o[d][4 * r4 + 3] * inv));
        *(uint2*)(orow + dd) = w;
      }
    if (g == 0) lse[((long)b * H + h) * Tn + qi] = (mrow + log2f(lrow)) / LOG2E;
  }
}

// dK, dV: a wave owns 32 keys; loop over the 64-query blocks that see them.
template <int HD>
__global__ void __launch_bounds__(256) attn_dkv_mfma(const bf16_t* qkv, const float* lse,
                                                     const bf16_t* dout, const float* D,
                                                     bf16_t* dqkv, int Tn, int H, int left,
                                                     float scale, float scale_log2) {
  constexpr int P = pitch_of<HD>(), NS = HD / 16, ND = HD / 32;
  __shared__ __attribute__((aligned(16))) bf16_t Qbuf[2][KB * P];
  __shared__ __attribute__((aligned(16))) bf16_t Gbuf[2][KB * P];
  __shared__ float Lbuf[2][KB], Dbuf[2][KB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int h = blockIdx.y, b = blockIdx.z;
  const long C = (long)H * HD, ld = 3 * C;
  const bf16_t* base = qkv + (long)b * Tn * ld;
  const bf16_t* gbase = dout + (long)b * Tn * C;
  const float* lrow = lse + ((long)b * H + h) * Tn;
  const float* drow = D + ((long)b * H + h) * Tn;
  const int kblk0 = blockIdx.x * 128;
  const int kw0 = kblk0 + wave * 32;
  const int kj = kw0 + c;  // this lane's key (as an operand column)

  bf16x8 kf[NS], vf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4 a{0, 0, 0, 0}, v{0, 0, 0, 0};
    if (kj < Tn) {
      a = *(const u32x4*)(base + (long)kj * ld + C + h * HD + 16 * s + 8 * g);
      v = *(const u32x4*)(base + (long)kj * ld + 2 * C + h * HD + 16 * s + 8 * g);
    }
    kf[s] = *(bf16x8*)&a;
    vf[s] = *(bf16x8*)&v;
  }
  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[d][r] = dv[d][r] = 0.f;

  const int klast = min(Tn - 1, kblk0 + 127);
  const int qend = left < 0 ? Tn - 1 : min(Tn - 1, klast + left);
  const int qstart = (kblk0 / KB) * KB;
  TileRegs<HD> rq, rg;
  float rl = 0.f, rd = 0.f;
  auto load_blk = [&](int q0) {
    tile_load<HD>(base + h * HD, ld, q0, Tn, rq);
    tile_load<HD>(gbase + h * HD, C, q0, Tn, rg);
    if (threadIdx.x < KB) {
      const int q = q0 + threadIdx.x;
      rl = q < Tn ? lrow[q] * LOG2E : 0.f;
      rd = q < Tn ? drow[q] : 0.f;
    }
  };
  auto store_blk = [&](int bb) {
    tile_store<HD>(rq, Qbuf[bb]);
    tile_store<HD>(rg, Gbuf[bb]);
    if (threadIdx.x < KB) {
      Lbuf[bb][threadIdx.x] = rl;
      Dbuf[bb][threadIdx.x] = rd;
    }
  };
  load_blk(qstart);
  store_blk(0);
  __syncthreads();
  int buf = 0;
  for (int qb0 = qstart; qb0 <= qend; qb0 += KB, buf ^= 1) {
    const bf16_t* Qs = Qbuf[buf];
    const bf16_t* Gs = Gbuf[buf];
    const float* Ls = Lbuf[buf];
    const float* Ds = Dbuf[buf];
    const bool more = qb0 + KB <= qend;
    if (more) load_blk(qb0 + KB);
    const bool skip = qb0 + KB - 1 < kw0 || (left >= 0 && qb0 > kw0 + 31 + left);
    if (!skip) {
    const bool full = qb0 >= kw0 + 31 && qb0 + KB - 1 < Tn && (left < 0 || qb0 + KB - 1 - kw0 <= left);
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<HD>(Qs, qq * 32, st, lane), kf[st], s,
                                                    0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<HD>(Gs, qq * 32, st, lane), vf[st],
                                                     dp, 0, 0, 0);
      }
      // s[r]: query qb0 + qq*32 + acc_row(r, g), key kj.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int ql = qq * 32 + acc_row(r, g);
        int qi = qb0 + ql;
        float p = (full || (qi < Tn && visible(qi, kj, left, Tn))) ? exp2f(s[r] * scale_log2 - Ls[ql])
                                                                   : 0.f;
        s[r] = p;
        dp[r] = p * (dp[r] - Ds[ql]);
      }
      // dV[key][d] += P^T[key][q] dO[q][d];  dK[key][d] += dS^T[key][q] Q[q][d]
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 pa = acc_slots(s, s2);
        bf16x8 da = acc_slots(dp, s2);
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              pa, tr_slots<HD>(Gs, d * 32, qq * 32 + 16 * s2, lane), dv[d], 0, 0, 0);
          dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              da, tr_slots<HD>(Qs, d * 32, qq * 32 + 16 * s2, lane), dk[d], 0, 0, 0);
        }
      }
    }
    }  // !skip
    if (more) store_blk(buf ^ 1);
    __syncthreads();
  }
  // dk[d][r]: key kw0 + acc_row(r, g), head dim d*32 + c.
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int key = kw0 + acc_row(r, g);
      if (key < Tn) {
        bf16_t* row = dqkv + ((long)b * Tn + key) * ld + h * HD + d * 32 + c;
        row[C] = f2bf(dk[d][r] * scale);
        row[2 * C] = f2bf(dv[d][r]);
      }
    }
}

// dQ: a wave owns 32 queries; loop over their key blocks.
template <int HD>
__global__ void __launch_bounds__(256) attn_dq_mfma(const bf16_t* qkv, const float* lse,
                                                    const bf16_t* dout, const float* D,
                                                    bf16_t* dqkv, int Tn, int H, int left,
                                                    float scale, float scale_log2) {
  constexpr int P = pitch_of<HD>(), NS = HD / 16, ND = HD / 32;
  __shared__ __attribute__((aligned(16))) bf16_t Kbuf[2][KB * P];
  __shared__ __attribute__((aligned(16))) bf16_t Vbuf[2][KB * P];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int h = blockIdx.y, b = blockIdx.z;
  const long C = (long)H * HD, ld = 3 * C;
  const bf16_t* base = qkv + (long)b * Tn * ld;
  const int qblk0 = blockIdx.x * 128;
  const int qw0 = qblk0 + wave * 32;
  const int qi = qw0 + c;

  bf16x8 qf[NS], gf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4 a{0, 0, 0, 0}, v{0, 0, 0, 0};
    if (qi < Tn) {
      a = *(const u32x4*)(base + (long)qi * ld + h * HD + 16 * s + 8 * g);
      v = *(const u32x4*)(dout + ((long)b * Tn + qi) * C + h * HD + 16 * s + 8 * g);
    }
    qf[s] = *(bf16x8*)&a;
    gf[s] = *(bf16x8*)&v;
  }
  const long r0 = ((long)b * H + h) * Tn;
  const float Lq = qi < Tn ? lse[r0 + qi] * LOG2E : 0.f;
  const float Dq = qi < Tn ? D[r0 + qi] : 0.f;
  f32x16 dq[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[d][r] = 0.f;

  const int qlast = min(Tn - 1, qblk0 + 127);
  const int kfirst = left < 0 ? 0 : max(0, qblk0 - left);
  const int kstart = (kfirst / KB) * KB;
  TileRegs<HD> rk, rv;
  tile_load<HD>(base + C + h * HD, ld, kstart, Tn, rk);
  tile_load<HD>(base + 2 * C + h * HD, ld, kstart, Tn, rv);
  tile_store<HD>(rk, Kbuf[0]);
  tile_store<HD>(rv, Vbuf[0]);
  __syncthreads();
  int buf = 0;
  for (int kb0 = kstart; kb0 <= qlast; kb0 += KB, buf ^= 1) {
    const bf16_t* Ks = Kbuf[buf];
    const bf16_t* Vs = Vbuf[buf];
    const bool more = kb0 + KB <= qlast;
    if (more) {
      tile_load<HD>(base + C + h * HD, ld, kb0 + KB, Tn, rk);
      tile_load<HD>(base + 2 * C + h * HD, ld, kb0 + KB, Tn, rv);
    }
    const bool skip = kb0 > qw0 + 31 || (left >= 0 && kb0 + KB - 1 < qw0 - left);
    if (!skip) {
    const bool full = kb0 + KB - 1 <= qw0 && qw0 + 31 < Tn && (left < 0 || qw0 + 31 - kb0 <= left);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<HD>(Ks, kk * 32, st, lane), qf[st], s,
                                                    0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<HD>(Vs, kk * 32, st, lane), gf[st],
                                                     dp, 0, 0, 0);
      }
      // s[r]: key kb0 + kk*32 + acc_row(r, g), query qi.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int j = kb0 + kk * 32 + acc_row(r, g);
        float p = (full || (qi < Tn && visible(qi, j, left, Tn))) ? exp2f(s[r] * scale_log2 - Lq)
                                                                  : 0.f;
        dp[r] = p * (dp[r] - Dq);
      }
      // dQ[q][d] += dS[q][key] K[key][d]
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 da = acc_slots(dp, s2);
#pragma unroll
        for (int d = 0; d < ND; ++d)
          dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              da, tr_slots<HD>(Ks, d * 32, kk * 32 + 16 * s2, lane), dq[d], 0, 0, 0);
      }
    }
    }  // !skip
    if (more) {
      tile_store<HD>(rk, Kbuf[buf ^ 1]);
      tile_store<HD>(rv, Vbuf[buf ^ 1]);
    }
    __syncthreads();
  }
  // dq[d][r]: query qw0 + acc_row(r, g), head dim d*32 + c.
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int q = qw0 + acc_row(r, g);
      if (q < Tn) dqkv[((long)b * Tn + q) * ld + h * HD + d * 32 + c] = f2bf(dq[d][r] * scale);
    }
}

template <int HD>
hipError_t launch_fwd(int B, int T, int H, int left, const void* qkv, void* out, float* lse,
                      hipStream_t s) {
  dim3 grid((unsigned)cdiv(T, 128), H, B);
  float sl2 = LOG2E / sqrtf((float)HD);
  attn_fwd_mfma<HD><<<grid, 256, 0, s>>>((const bf16_t*)qkv, (bf16_t*)out, lse, T, H, left, sl2);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_bwd(int B, int T, int H, int left, const void* qkv, const float* lse,
                      const void* dout, const float* D, void* dqkv, hipStream_t s) {
  dim3 grid((unsigned)cdiv(T, 128), H, B);
  float sc = 1.f / sqrtf((float)HD);
  float sl2 = sc * LOG2E;
  attn_dkv_mfma<HD><<<grid, 256, 0, s>>>((const bf16_t*)qkv, lse, (const bf16_t*)dout, D,
                                         (bf16_t*)dqkv, T, H, left, sc, sl2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_dq_mfma<HD><<<grid, 256, 0, s>>>((const bf16_t*)qkv, lse, (const bf16_t*)dout, D,
                                        (bf16_t*)dqkv, T, H, left, sc, sl2);
  return hipGetLastError();
}

}  // namespace

bool attention_supported(int prec, int hd) {
  if (prec == GPT_BF16) return hd == 32 || hd == 64 || hd == 128;
  return hd >= 1 && hd <= 128;
}

hipError_t attention_fwd(int prec, int B, int T, int H, int hd, int left, const void* qkv,
                         void* out, float* lse, hipStream_t s) {
  if ((long)B * T * H == 0) return hipSuccess;
  if (!attention_supported(prec, hd)) return hipErrorInvalidValue;
  if (prec == GPT_BF16) {
    if (hd == 32) return launch_fwd<32>(B, T, H, left, qkv, out, lse, s);
    if (hd == 64) return launch_fwd<64>(B, T, H, left, qkv, out, lse, s);
    return launch_fwd<128>(B, T, H, left, qkv, out, lse, s);
  }
  long waves = (long)B * H * T;
  attn_fwd_rows<float><<<(unsigned)cdiv(waves, 4), 256, 0, s>>>(
      (const float*)qkv, (float*)out, lse, B, T, H, hd, left, 1.f / sqrtf((float)hd));
  return hipGetLastError();
}

hipError_t attention_bwd(int prec, int B, int T, int H, int hd, int left, const void* qkv,
                         const void* out, const float* lse, const void* dout, void* dqkv,
                         float* dvec, hipStream_t s) {
  if ((long)B * T * H == 0) return hipSuccess;
  if (!attention_supported(prec, hd)) return hipErrorInvalidValue;
  long rows = (long)B * T * H;
  if (prec == GPT_BF16) {
    const long M = (long)B * T;
    const unsigned g = (unsigned)cdiv(M, 4);
    if (hd == 32)
      attn_dvec_bf16<32><<<g, 256, 0, s>>>((const bf16_t*)out, (const bf16_t*)dout, dvec, (int)M, T, H);
    else if (hd == 64)
      attn_dvec_bf16<64><<<g, 256, 0, s>>>((const bf16_t*)out, (const bf16_t*)dout, dvec, (int)M, T, H);
    else
      attn_dvec_bf16<128><<<g, 256, 0, s>>>((const bf16_t*)out, (const bf16_t*)dout, dvec, (int)M, T, H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (hd == 32) return launch_bwd<32>(B, T, H, left, qkv, lse, dout, dvec, dqkv, s);
    if (hd == 64) return launch_bwd<64>(B, T, H, left, qkv, lse, dout, dvec, dqkv, s);
    return launch_bwd<128>(B, T, H, left, qkv, lse, dout, dvec, dqkv, s);
  }
  attn_dvec<float><<<(unsigned)cdiv(rows, 256), 256, 0, s>>>((const float*)out,
                                                             (const float*)dout, dvec, B, T, H, hd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float sc = 1.f / sqrtf((float)hd);
  attn_dq_rows<float><<<(unsigned)cdiv(rows, 4), 256, 0, s>>>(
      (const float*)qkv, lse, (const float*)dout, dvec, (float*)dqkv, B, T, H, hd, left, sc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_dkv_rows<float><<<(unsigned)cdiv(rows, 4), 256, 0, s>>>(
      (const float*)qkv, lse, (const float*)dout, dvec, (float*)dqkv, B, T, H, hd, left, sc);
  return hipGetLastError();
}

}  // namespace gpt
