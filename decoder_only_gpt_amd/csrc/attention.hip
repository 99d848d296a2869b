// Causal multi-head self-attention with an optional left window, forward and
// backward.
//
// What is computed (nanoGPT README, "quick start": a six-layer, six-head model;
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
//   A wave raises its priority for its MFMA bursts (s_setprio) and drops it
//   for the softmax rebuild between them, so the SIMD's other wave, in its
//   VALU phase, fills the issue slots the matrix unit leaves (3% faster; the
//   forward, at three waves per SIMD, is slower with it and has none).
// fp32 path: one wave per (query) or (key) row with exact fp32 arithmetic.

#include "common.h"
#include "kernels.h"

#include <mutex>
#include <type_traits>
#include <vector>

namespace gpt {

// Device scratch of the allocation-free backward entry point: D and the
// log-sum-exp in log2 units, 2 * B*H*T floats.  Every GPU the library runs on
// holds its own copy until the process ends; host code reaches it only
// through the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[ATTN_SCRATCH_FLOATS];

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

// D[b,h,i] = sum_d dO[i,d] * O[i,d]  (one thread per (row, head)); the bf16
// path computes it inside the dQ kernel.
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
//
// Tiles of 64 rows x HD head dims are fetched straight into LDS with buffer
// loads (buffer_load_dwordx4 ... lds): one wave instruction fills a contiguous
// 1 KB block (lane l -> bytes 16 l), so tile rows are stored densely (2 HD
// bytes each) and the 16-byte chunk index is XOR-swizzled through the source
// address each lane picks.  Rows at or past the sequence end get an offset
// outside the buffer and read zeros.  Tile t + 1 is in flight while tile t is
// multiplied; one barrier per tile.
// ---------------------------------------------------------------------------
constexpr int KB = 64;  // rows per LDS tile: keys (forward, dQ) or queries (dK/dV)

typedef __attribute__((address_space(3))) void lds_void;

// Chunk swizzle of tile row r: the 16 rows of a 16-byte fragment read and the
// 4 rows x 64 bytes of a transpose read land on distinct 16-byte bank groups
// (64 banks of 4 bytes).
template <int HD> __device__ __forceinline__ int swz(int r) {
  if constexpr (HD == 32) return (r >> 2) & 3;
  else if constexpr (HD == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}
// Element offset of (row r, head dim col) in a swizzled tile.
template <int HD> __device__ __forceinline__ int toff(int r, int col) {
  return r * HD + (((col >> 3) ^ swz<HD>(r)) << 3) + (col & 7);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// max / sum of a value and its partner 32 lanes away (v_permlane32_swap: one
// VALU op, where a shuffle would go through the LDS crossbar); both halves of
// the wave get the identical result.
__device__ __forceinline__ float swap32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// This wave's share of the loads of rows [row0, row0 + 64), columns
// [col0, col0 + HD) of a bf16 matrix (leading dimension ld) into a tile.
template <int HD>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, long ld, int col0, int row0,
                                         int nrows, bf16_t* lds, int wave, int lane) {
  constexpr int NC = HD / 8, RPB = 64 / NC, NB = KB / RPB;  // chunks / row, rows / block, blocks
#pragma unroll
  for (int i = 0; i < NB / 4; ++i) {
    const int blk = wave * (NB / 4) + i;
    const int r = blk * RPB + lane / NC;
    const int chunk = (lane % NC) ^ swz<HD>(r);
    const unsigned off = row0 + r < nrows
                             ? (unsigned)(((long)(row0 + r) * ld + col0 + chunk * 8) * 2)
                             : 0x80000000u;
    // Issued from inline asm (M0 = the block's LDS address): the compiler's
    // wait insertion would otherwise put a vmcnt(0) after these loads, ahead
    // of the current stage's fragment reads, and the next tile would never
    // load while this one is multiplied.  Every loop waits vmcnt(0) and
    // synchronises before it reads a stage or refills the other one.
    const unsigned m0v = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds + blk * 512));
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0v), "v"(off), "s"(rs)
                 : "memory", "m0");
  }
}

// MFMA operand fragment whose lane index (lane % 32) runs along the tile rows:
// row r0 + lane % 32, head dims 16 st + 8 (lane / 32) + 0..7.
template <int HD>
__device__ __forceinline__ bf16x8 row_frag(const bf16_t* t, int r0, int st, int lane) {
  return *(const bf16x8*)(t + toff<HD>(r0 + (lane & 31), 16 * st + 8 * (lane >> 5)));
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
  const int s = lane & 15, grp = lane >> 4;
  const int col = c0 + 16 * (grp & 1) + 4 * (s & 3);
  const int row = base + 4 * (grp >> 1) + (s >> 2);
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + toff<HD>(row, col)));
  v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + toff<HD>(row + 8, col)));
  v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return *(bf16x8*)&v;
}

// 8 accumulator values r = 8*s2 .. 8*s2+7 of a 32x32 block as a bf16 operand.
__device__ __forceinline__ bf16x8 acc_slots(const f32x16& acc, int s2) {
  u32x4 v{pack_bf2(acc[8 * s2 + 0], acc[8 * s2 + 1]), pack_bf2(acc[8 * s2 + 2], acc[8 * s2 + 3]),
          pack_bf2(acc[8 * s2 + 4], acc[8 * s2 + 5]), pack_bf2(acc[8 * s2 + 6], acc[8 * s2 + 7])};
  return *(bf16x8*)&v;
}

// Row of accumulator register r for lane half g of a 32x32 MFMA block.
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Store a [32 dims][32 columns] accumulator block (lane % 32 = column) as
// bf16 into row `dst` (this lane's column), head dims d0 + acc_row(r, g).
__device__ __forceinline__ void store_dims(bf16_t* dst, int d0, const f32x16& a, float mul, int g) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *(uint2*)(dst + d0 + 8 * i + 4 * g) =
        make_uint2(pack_bf2(a[4 * i] * mul, a[4 * i + 1] * mul),
                   pack_bf2(a[4 * i + 2] * mul, a[4 * i + 3] * mul));
}

// Store a wave's [32 rows][HD] output block, held as HD / 32 accumulators
// (acc[d][r]: head dim d * 32 + acc_row(r, g) of row lane % 32), as bf16 rows
// dst + i * ldr (i < nrows), each value times this lane's `mul`.  The block is
// staged through the wave's LDS slice `st` (32 rows of HD + 8 elements, the
// pad spreading the rows over the banks) so that every row leaves as whole
// 16-byte chunks, HD / 8 consecutive lanes per row: the stores write full
// cache lines instead of a 16-byte piece of 32 rows per instruction.  The
// caller makes sure no other wave still reads `st`.
template <int HD>
__device__ __forceinline__ void store_rows(bf16_t* dst, long ldr, int nrows, const f32x16* acc,
                                           float mul, bf16_t* st, int lane) {
  constexpr int ND = HD / 32, P = HD + 8, LPR = HD / 8, RPP = 64 / LPR;
  const int c = lane & 31, g = lane >> 5;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(uint2*)(st + c * P + d * 32 + 8 * i + 4 * g) =
          make_uint2(pack_bf2(acc[d][4 * i] * mul, acc[d][4 * i + 1] * mul),
                     pack_bf2(acc[d][4 * i + 2] * mul, acc[d][4 * i + 3] * mul));
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the slice is written
#pragma unroll
  for (int pass = 0; pass < 32 / RPP; ++pass) {
    const int r = pass * RPP + lane / LPR, ch = lane % LPR;
    const u32x4 v = *(const u32x4*)(st + r * P + ch * 8);
    if (r < nrows) *(u32x4*)(dst + (long)r * ldr + ch * 8) = v;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the slice is reused
}
template <int HD> constexpr int store_slice_elems() { return 32 * (HD + 8); }

template <bool B> struct Mask { static constexpr bool value = B; };

// Forward: 128 queries of one (batch, head) per workgroup, 32 per wave.
template <int HD>
__global__ void __launch_bounds__(256, HD == 128 ? 1 : 2)
    attn_fwd_mfma(const bf16_t* qkv, bf16_t* out, float* lse, int Tn, int H, int left,
                  float scale_log2) {
  constexpr int NS = HD / 16, ND = HD / 32;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][KB * HD];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][KB * HD];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, c = lane & 31;
  const int h = blockIdx.x % H, b = blockIdx.x / H;
  const long C = (long)H * HD, ld = 3 * C;
  const bf16_t* base = qkv + (long)b * Tn * ld;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (long)Tn * ld * 2);
  const int qblk0 = (gridDim.y - 1 - blockIdx.y) * 128;  // longest key ranges first
  const int qw0 = qblk0 + wave * 32;
  const int qi = qw0 + c;  // this lane's query

  bf16x8 qf[NS];  // this lane's query row qi, head dims 16 s + 8 g .. (filled below)
  f32x16 o[ND];  // O^T: head dim d * 32 + acc_row(r, g), query qi
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = f32x16{};
  float mrow = -1e30f, lrow = 0.f;  // running max (log2 units) and sum

  const int qlast = min(Tn - 1, qblk0 + 127);
  const int kstart = left < 0 ? 0 : (max(0, qblk0 - left) / KB) * KB;

  auto step = [&](const bf16_t* Kt, const bf16_t* Vt, int kb0, auto mask) {
    constexpr bool MASK = decltype(mask)::value;
    f32x16 s[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      s[kk] = f32x16{};
#pragma unroll
      for (int st = 0; st < NS; ++st)
        s[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<HD>(Kt, kk * 32, st, lane), qf[st],
                                                        s[kk], 0, 0, 0);
    }
    // s[kk][r]: key kb0 + kk * 32 + acc_row(r, g), query qi (raw scores)
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (MASK) {
          const int j = kb0 + kk * 32 + acc_row(r, g);
          if (!visible(qi, j, left, Tn)) s[kk][r] = -INFINITY;
        }
        mx = fmaxf(mx, s[kk][r]);
      }
    // The two halves of the wave hold the two 16-key halves of each 32-key
    // block for the same query: combined by one lane swap.
    mx = swap32_max(mx);
    // Lazy rescaling: the running maximum (log2 units) is raised, and O and
    // the sum rescaled, only when some query's block maximum exceeds it by
    // more than 8; otherwise the exponents use the stale maximum, so every
    // p <= 2^8 and O / sum is unchanged mathematically.
    const float mcand = mx * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mcand > mrow + 8.f) != 0) {
      const float mnew = fmaxf(mrow, mcand);
      const float alpha = __builtin_amdgcn_exp2f(mrow - mnew);
      lrow *= alpha;
#pragma unroll
      for (int d = 0; d < ND; ++d) o[d] *= alpha;
      mrow = mnew;
    }
    float ls = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kk][r], scale_log2, -mrow));
        s[kk][r] = p;
        ls += p;
      }
    lrow += swap32_sum(ls);
    // O^T[d][q] += V^T[d][key] P^T[key][q]
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 pf = acc_slots(s[kk], s2);
#pragma unroll
        for (int d = 0; d < ND; ++d)
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tr_slots<HD>(Vt, d * 32, kk * 32 + 16 * s2, lane), pf, o[d], 0, 0, 0);
      }
  };

  dma_tile<HD>(rs, ld, C + h * HD, kstart, Tn, Ks[0], wave, lane);
  dma_tile<HD>(rs, ld, 2 * C + h * HD, kstart, Tn, Vs[0], wave, lane);
  // The workgroup's 128 query rows pass through the second K and V stages
  // (free until the loop first refills them) as whole-row loads; each wave
  // then reads its 32 queries' fragments (zero rows past the sequence end).
  dma_tile<HD>(rs, ld, h * HD, qblk0, Tn, Ks[1], wave, lane);
  dma_tile<HD>(rs, ld, h * HD, qblk0 + 64, Tn, Vs[1], wave, lane);
  __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's loads landed
  __syncthreads();                     // ... and every other wave's
#pragma unroll
  for (int s = 0; s < NS; ++s)
    qf[s] = row_frag<HD>(wave < 2 ? Ks[1] : Vs[1], (wave & 1) * 32, s, lane);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): read before the stages are refilled
  int buf = 0;
  for (int kb0 = kstart; kb0 <= qlast; kb0 += KB, buf ^= 1) {
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's share of tile kb0 landed
    __syncthreads();                     // ... and every other wave's
    if (kb0 + KB <= qlast) {
      dma_tile<HD>(rs, ld, C + h * HD, kb0 + KB, Tn, Ks[buf ^ 1], wave, lane);
      dma_tile<HD>(rs, ld, 2 * C + h * HD, kb0 + KB, Tn, Vs[buf ^ 1], wave, lane);
    }
    const bool skip = kb0 > qw0 + 31 || (left >= 0 && kb0 + KB - 1 < qw0 - left);
    if (skip) continue;
    // every (query, key) pair of this wave and block visible: no per-element mask
    const bool full =
        kb0 + KB - 1 <= qw0 && qw0 + 31 < Tn && (left < 0 || qw0 + 31 - kb0 <= left);
    if (full) step(Ks[buf], Vs[buf], kb0, Mask<false>{});
    else step(Ks[buf], Vs[buf], kb0, Mask<true>{});
  }
  // (Staging these rows through LDS, as the backward kernels do, is slower here.)
  if (qi < Tn) {
    const float inv = 1.f / lrow;
    bf16_t* orow = out + ((long)b * Tn + qi) * C + h * HD;
#pragma unroll
    for (int d = 0; d < ND; ++d) store_dims(orow, d * 32, o[d], inv, g);
    if (g == 0) lse[((long)b * H + h) * Tn + qi] = (mrow + log2f(lrow)) / LOG2E;
  }
}

// Scheduling of one phase of a software-pipelined tile: MFMA i of the phase,
// then its share of the LDS reads (of the next phase's fragments) and of the
// VALU work, for i = 0 .. NM - 1.
template <int NM, int NDS, int NV, int I = 0> __device__ __forceinline__ void phase_pattern() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int ds = NDS / NM + (I < NDS % NM ? 1 : 0);
    constexpr int nv = NV / NM + (I < NV % NM ? 1 : 0);
    if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds, 0);
    if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x002, nv, 0);
    phase_pattern<NM, NDS, NV, I + 1>();
  }
}

// dK, dV: 128 keys of one (batch, head) per workgroup, 32 per wave; the
// workgroup walks 128-query tiles of Q and dO (QT rows each, two LDS stages,
// with the per-query L2 and D).  L2 is the saved log-sum-exp in log2 units,
// D[q] = sum_d dO[q][d] O[q][d].  A tile whose (query, key) pairs are all
// visible runs its four 32-query sub-blocks without masks or per-sub-block
// branches; other tiles (diagonal, window edge, sequence end) take a
// per-sub-block masked path.  (A software pipeline like the dQ kernel's needs
// more registers than two waves per SIMD leave here: it spills.)
constexpr int QT = 128;  // queries per LDS tile of the dK/dV kernel

template <int HD>
__global__ void __launch_bounds__(256, HD == 128 ? 1 : 2)
    attn_dkv_mfma(const bf16_t* qkv, const float* L2, const bf16_t* dout, const float* D,
                  bf16_t* dqkv, int Tn, int H, int left, float scale, float scale_log2) {
  constexpr int NS = HD / 16, ND = HD / 32;
  __shared__ __attribute__((aligned(16))) bf16_t Qs[2][QT * HD];
  __shared__ __attribute__((aligned(16))) bf16_t Gs[2][QT * HD];
  __shared__ __attribute__((aligned(16))) float Ls[2][QT];
  __shared__ __attribute__((aligned(16))) float Ds[2][QT];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, c = lane & 31;
  const int h = blockIdx.x % H, b = blockIdx.x / H;
  const long C = (long)H * HD, ld = 3 * C;
  const bf16_t* base = qkv + (long)b * Tn * ld;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(base, (long)Tn * ld * 2);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(dout + (long)b * Tn * C, (long)Tn * C * 2);
  const float* lrow = L2 + ((long)b * H + h) * Tn;
  const float* drow = D + ((long)b * H + h) * Tn;
  const int kblk0 = blockIdx.y * 128;  // earliest keys (most queries) first
  const int kw0 = kblk0 + wave * 32;
  const int kj = kw0 + c;  // this lane's key (operand column)

  bf16x8 kf[NS], vf[NS];  // this lane's key row kj, head dims 16 s + 8 g .. (filled below)
  f32x16 dk[ND], dv[ND];  // dK^T, dV^T: head dim d * 32 + acc_row(r, g), key kj
#pragma unroll
  for (int d = 0; d < ND; ++d) dk[d] = dv[d] = f32x16{};

  const int klast = min(Tn - 1, kblk0 + 127);
  const int qend = left < 0 ? Tn - 1 : min(Tn - 1, klast + left);

  // S and dP of the 32 queries at tile row r0 (s[r], dp[r]: query r0 +
  // acc_row(r, g), key kj), from fragments qr / gr.
  auto sdp = [&](f32x16& s, f32x16& dp, const bf16x8* qr, const bf16x8* gr) {
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qr[st], kf[st], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gr[st], vf[st], dp, 0, 0, 0);
    }
  };
  auto rows = [&](bf16x8* qr, bf16x8* gr, const bf16_t* Qt, const bf16_t* Gt, int r0) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      qr[st] = row_frag<HD>(Qt, r0, st, lane);
      gr[st] = row_frag<HD>(Gt, r0, st, lane);
    }
  };
  // P = exp2(S log2e / sqrt(hd) - L2), dS = P (dP - D) as bf16 operands; MASK
  // zeroes P outside the visible band (qb = the sub-block's first query).
  auto soft = [&](f32x16& s, f32x16& dp, const float* Lt, const float* Dt, int r0, bf16x8* pa,
                  bf16x8* da, auto mask, int qb) {
    constexpr bool MASK = decltype(mask)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ql = r0 + 8 * i + 4 * g;
      const f32x4 lv = *(const f32x4*)(Lt + ql);
      const f32x4 dd = *(const f32x4*)(Dt + ql);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float p = __builtin_amdgcn_exp2f(fmaf(s[4 * i + j], scale_log2, -lv[j]));
        if constexpr (MASK) {
          const int qi = qb + 8 * i + 4 * g + j;
          if (qi >= Tn || !visible(qi, kj, left, Tn)) p = 0.f;
        }
        s[4 * i + j] = p;
        dp[4 * i + j] = p * (dp[4 * i + j] - dd[j]);
      }
    }
    pa[0] = acc_slots(s, 0);
    pa[1] = acc_slots(s, 1);
    da[0] = acc_slots(dp, 0);
    da[1] = acc_slots(dp, 1);
  };
  // dV^T[d][key] += dO^T[d][q] P[q][key];  dK^T[d][key] += Q^T[d][q] dS[q][key]
  // over the 32 queries at tile row r0; the transposed fragments of each
  // 16-query half are read just before its MFMAs.
  auto dvk = [&](const bf16_t* Qt, const bf16_t* Gt, int r0, const bf16x8* pa, const bf16x8* da) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 tg[ND], tq[ND];
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        tg[d] = tr_slots<HD>(Gt, d * 32, r0 + 16 * s2, lane);
        tq[d] = tr_slots<HD>(Qt, d * 32, r0 + 16 * s2, lane);
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tg[d], pa[s2], dv[d], 0, 0, 0);
        dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[d], da[s2], dk[d], 0, 0, 0);
      }
    }
  };

  // Per-query scalars travel through registers (one per thread of the first two waves).
  float rl = 0.f, rd = 0.f;
  auto fetch = [&](int q0, int bb) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      dma_tile<HD>(rq, ld, h * HD, q0 + 64 * half, Tn, Qs[bb] + 64 * half * HD, wave, lane);
      dma_tile<HD>(rg, C, h * HD, q0 + 64 * half, Tn, Gs[bb] + 64 * half * HD, wave, lane);
    }
    if (threadIdx.x < QT) {
      const int q = q0 + threadIdx.x;
      rl = q < Tn ? lrow[q] : 0.f;
      rd = q < Tn ? drow[q] : 0.f;
    }
  };
  fetch(kblk0, 0);
  // The workgroup's 128 K and V rows pass through the second Q / dO stage
  // (free until the loop first refills it) as whole-row loads; each wave then
  // reads its 32 keys' fragments (zero rows past the sequence end).
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    dma_tile<HD>(rq, ld, C + h * HD, kblk0 + 64 * half, Tn, Qs[1] + 64 * half * HD, wave, lane);
    dma_tile<HD>(rq, ld, 2 * C + h * HD, kblk0 + 64 * half, Tn, Gs[1] + 64 * half * HD, wave, lane);
  }
  if (threadIdx.x < QT) {
    Ls[0][threadIdx.x] = rl;
    Ds[0][threadIdx.x] = rd;
  }
  __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's loads landed
  __syncthreads();                     // ... and every other wave's
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kf[s] = row_frag<HD>(Qs[1], wave * 32, s, lane);
    vf[s] = row_frag<HD>(Gs[1], wave * 32, s, lane);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): read before the stage is refilled
  int buf = 0;
  for (int qb0 = kblk0; qb0 <= qend; qb0 += QT, buf ^= 1) {
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's share of block qb0 landed
    __syncthreads();                     // ... and every other wave's (tiles and scalars)
    const bool more = qb0 + QT <= qend;
    if (more) fetch(qb0 + QT, buf ^ 1);
    const bf16_t* Qt = Qs[buf];
    const bf16_t* Gt = Gs[buf];
    const float* Lt = Ls[buf];
    const float* Dt = Ds[buf];
    // every (query, key) pair of the workgroup visible in this tile: uniform branch
    const bool full = qb0 >= kblk0 + 127 && qb0 + QT <= Tn &&
                      (left < 0 || qb0 + QT - 1 - kblk0 <= left);
    if (full) {
      f32x16 s, dp;
      bf16x8 qr[NS], gr[NS], pa[2], da[2];
#pragma unroll 1
      for (int j = 0; j < QT / 32; ++j) {
        rows(qr, gr, Qt, Gt, 32 * j);
        sdp(s, dp, qr, gr);
        soft(s, dp, Lt, Dt, 32 * j, pa, da, Mask<false>{}, 0);
        dvk(Qt, Gt, 32 * j, pa, da);
      }
    } else {
#pragma unroll 1
      for (int j = 0; j < QT / 32; ++j) {
        const int qb = qb0 + 32 * j;
        const bool skip = qb + 31 < kw0 || (left >= 0 && qb > kw0 + 31 + left) || qb >= Tn;
        if (skip) continue;
        f32x16 s, dp;
        bf16x8 qr[NS], gr[NS], pa[2], da[2];
        rows(qr, gr, Qt, Gt, 32 * j);
        sdp(s, dp, qr, gr);
        soft(s, dp, Lt, Dt, 32 * j, pa, da, Mask<true>{}, qb);
        dvk(Qt, Gt, 32 * j, pa, da);
      }
    }
    if (more && threadIdx.x < QT) {
      Ls[buf ^ 1][threadIdx.x] = rl;
      Ds[buf ^ 1][threadIdx.x] = rd;
    }
  }
  __syncthreads();  // every wave is done with the Q / dO tiles: they become output slices
  static_assert(4 * store_slice_elems<HD>() <= 2 * QT * HD, "output slices fit the Q tiles");
  {
    bf16_t* const st = &Qs[0][0] + wave * store_slice_elems<HD>();
    bf16_t* const row = dqkv + ((long)b * Tn + kw0) * ld + h * HD;
    const int nrows = min(32, Tn - kw0);
    store_rows<HD>(row + C, ld, nrows, dk, scale, st, lane);
    store_rows<HD>(row + 2 * C, ld, nrows, dv, 1.f, st, lane);
  }
}

// dQ: 128 queries of one (batch, head) per workgroup, 32 per wave; the
// workgroup walks 128-key tiles of K and V (KT rows each, two LDS stages).
// A tile whose 128 x 128 (query, key) pairs are all visible is multiplied in
// a software pipeline over its four 32-key sub-blocks: the MFMAs of S and dP
// for sub-block n + 1 and of dQ for sub-block n - 1 are issued between the
// VALU instructions that rebuild P and dS for sub-block n, so the matrix unit
// and the ALUs work at the same time within one wave.  Tiles on the diagonal,
// at a window edge or past the sequence end take a per-sub-block masked path.
constexpr int KT = 128;  // keys per LDS tile of the dQ kernel

template <int HD>
__global__ void __launch_bounds__(256, HD == 128 ? 1 : 2)
    attn_dq_mfma(const bf16_t* qkv, const float* lse, const bf16_t* out, const bf16_t* dout,
                 float* D, float* L2, bf16_t* dqkv, int Tn, int H, int left, float scale,
                 float scale_log2) {
  constexpr int NS = HD / 16, ND = HD / 32;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][KT * HD];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][KT * HD];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, c = lane & 31;
  const int h = blockIdx.x % H, b = blockIdx.x / H;
  const long C = (long)H * HD, ld = 3 * C;
  const bf16_t* base = qkv + (long)b * Tn * ld;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (long)Tn * ld * 2);
  const int qblk0 = (gridDim.y - 1 - blockIdx.y) * 128;  // longest key ranges first
  const int qw0 = qblk0 + wave * 32;
  const int qi = qw0 + c;
  const int qlast = min(Tn - 1, qblk0 + 127);
  const int kstart = left < 0 ? 0 : (max(0, qblk0 - left) / KT) * KT;
  auto fetch = [&](int k0, int bb) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      dma_tile<HD>(rs, ld, C + h * HD, k0 + 64 * half, Tn, Ks[bb] + 64 * half * HD, wave, lane);
      dma_tile<HD>(rs, ld, 2 * C + h * HD, k0 + 64 * half, Tn, Vs[bb] + 64 * half * HD, wave, lane);
    }
  };
  // The first key tile is requested before this wave's own rows, so the two
  // memory latencies overlap instead of adding up.
  fetch(kstart, 0);
  // The workgroup's 128 Q and dO rows pass through the second K / V stage
  // (free until the loop first refills it) as whole-row loads; each wave then
  // reads its 32 queries' fragments (zero rows past the sequence end).  O,
  // needed only for D, is read straight into registers.
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(dout + (long)b * Tn * C, (long)Tn * C * 2);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    dma_tile<HD>(rs, ld, h * HD, qblk0 + 64 * half, Tn, Ks[1] + 64 * half * HD, wave, lane);
    dma_tile<HD>(rg, C, h * HD, qblk0 + 64 * half, Tn, Vs[1] + 64 * half * HD, wave, lane);
  }
  u32x4 orow[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    orow[s] = u32x4{0, 0, 0, 0};
    if (qi < Tn) orow[s] = *(const u32x4*)(out + ((long)b * Tn + qi) * C + h * HD + 16 * s + 8 * g);
  }
  __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's loads landed
  __syncthreads();                     // ... and every other wave's
  bf16x8 qf[NS], gf[NS];
  float dpart = 0.f;  // this lane's share of D = sum_d dO O for its query
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = row_frag<HD>(Ks[1], wave * 32, s, lane);
    gf[s] = row_frag<HD>(Vs[1], wave * 32, s, lane);
    const u32x4 v = *(const u32x4*)&gf[s], o = orow[s];
#pragma unroll
    for (int k = 0; k < 4; ++k) dpart += bf_lo(o[k]) * bf_lo(v[k]) + bf_hi(o[k]) * bf_hi(v[k]);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): read before the stage is refilled
  // Lanes c and c + 32 hold the two halves of query qi's head dims; the sum
  // and the log-sum-exp in log2 units also go to D and L2 for the dK/dV kernel.
  const long r0 = ((long)b * H + h) * Tn;
  const float Dq = dpart + __shfl_xor(dpart, 32, 64);
  const float Lq = qi < Tn ? lse[r0 + qi] * LOG2E : 0.f;
  if (g == 0 && qi < Tn) {
    D[r0 + qi] = Dq;
    L2[r0 + qi] = Lq;
  }
  f32x16 dq[ND];  // dQ^T: head dim d * 32 + acc_row(r, g), query qi
#pragma unroll
  for (int d = 0; d < ND; ++d) dq[d] = f32x16{};

  // S^T and dP^T of the 32-key sub-block at tile row kr: s[r], dp[r] hold key
  // kr + acc_row(r, g) for query qi.
  auto sdp = [&](f32x16& s, f32x16& dp, const bf16_t* Kt, const bf16_t* Vt, int kr) {
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<HD>(Kt, kr, st, lane), qf[st], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<HD>(Vt, kr, st, lane), gf[st], dp, 0, 0,
                                                   0);
    }
  };
  // P = exp2(S log2e / sqrt(hd) - L2), dS = P (dP - D), as two bf16 operands.
  auto soft = [&](const f32x16& s, const f32x16& dp, bf16x8* da) {
    f32x16 ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -Lq));
      ds[r] = p * (dp[r] - Dq);
    }
    da[0] = acc_slots(ds, 0);
    da[1] = acc_slots(ds, 1);
  };
  // dQ^T[d][q] += K^T[d][key] dS^T[key][q] over the sub-block at tile row kr.
  auto dqm = [&](const bf16x8* da, const bf16_t* Kt, int kr) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int d = 0; d < ND; ++d)
        dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_slots<HD>(Kt, d * 32, kr + 16 * s2, lane),
                                                        da[s2], dq[d], 0, 0, 0);
  };
  // One masked 32-key sub-block (diagonal, window edge, sequence end).
  auto masked = [&](const bf16_t* Kt, const bf16_t* Vt, int kr, int kb) {
    f32x16 s, dp;
    sdp(s, dp, Kt, Vt, kr);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -Lq));
      if (!visible(qi, kb + acc_row(r, g), left, Tn)) p = 0.f;
      dp[r] = p * (dp[r] - Dq);
    }
    const bf16x8 da[2] = {acc_slots(dp, 0), acc_slots(dp, 1)};
    dqm(da, Kt, kr);
  };
  // Scheduling pattern of a pipeline phase: the LDS reads first, then each
  // MFMA followed by an equal share of the VALU work.
  constexpr int SDP_M = 2 * NS, DQ_M = 2 * ND;       // MFMAs of sdp / dqm
  constexpr int SDP_R = 2 * NS, DQ_R = 4 * ND;       // LDS read instructions
  constexpr int SOFT_V = 16 * 4 + 8;                 // VALU instructions of soft
  int buf = 0;
  for (int kb0 = kstart; kb0 <= qlast; kb0 += KT, buf ^= 1) {
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's share of tile kb0 landed
    __syncthreads();                     // ... and every other wave's
    if (kb0 + KT <= qlast) fetch(kb0 + KT, buf ^ 1);
    const bf16_t* Kt = Ks[buf];
    const bf16_t* Vt = Vs[buf];
    // every (query, key) pair of the workgroup visible in this tile: uniform branch
    const bool full = kb0 + KT - 1 <= qblk0 && qblk0 + 127 < Tn &&
                      (left < 0 || qblk0 + 127 - kb0 <= left);
    if (full) {
      // Fragments are read one phase ahead of the MFMAs that use them, each
      // read issued right after the MFMA that frees its registers.
      f32x16 s0, p0, s1, p1;
      bf16x8 a0[2], a1[2], kr[NS], vr[NS], tf[2][ND];
      auto rows = [&](int r0) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          kr[st] = row_frag<HD>(Kt, r0, st, lane);
          vr[st] = row_frag<HD>(Vt, r0, st, lane);
        }
      };
      auto trs = [&](int r0) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int d = 0; d < ND; ++d) tf[s2][d] = tr_slots<HD>(Kt, d * 32, r0 + 16 * s2, lane);
      };
      auto sdp_m = [&](f32x16& s, f32x16& dp) {
        s = f32x16{};
        dp = f32x16{};
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[st], qf[st], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[st], gf[st], dp, 0, 0, 0);
        }
      };
      auto dqm_m = [&](const bf16x8* da) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int d = 0; d < ND; ++d)
            dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[s2][d], da[s2], dq[d], 0, 0, 0);
      };
      rows(0);
      __builtin_amdgcn_sched_barrier(0);
      sdp_m(s0, p0);
      rows(32);
      __builtin_amdgcn_sched_barrier(0);
      // phase 1: S, dP of sub-block 1; P, dS of 0
      sdp_m(s1, p1);
      trs(0);
      rows(64);
      soft(s0, p0, a0);
      phase_pattern<SDP_M, SDP_R + DQ_R, SOFT_V>();
      __builtin_amdgcn_sched_barrier(0);
      // phase 2: dQ of 0, S, dP of 2; P, dS of 1
      dqm_m(a0);
      trs(32);
      sdp_m(s0, p0);
      rows(96);
      soft(s1, p1, a1);
      phase_pattern<SDP_M + DQ_M, SDP_R + DQ_R, SOFT_V>();
      __builtin_amdgcn_sched_barrier(0);
      // phase 3: dQ of 1, S, dP of 3; P, dS of 2
      dqm_m(a1);
      trs(64);
      sdp_m(s1, p1);
      soft(s0, p0, a0);
      phase_pattern<SDP_M + DQ_M, DQ_R, SOFT_V>();
      __builtin_amdgcn_sched_barrier(0);
      // phase 4: dQ of 2; P, dS of 3
      dqm_m(a0);
      trs(96);
      soft(s1, p1, a1);
      phase_pattern<DQ_M, DQ_R, SOFT_V>();
      __builtin_amdgcn_sched_barrier(0);
      // phase 5: dQ of 3
      dqm_m(a1);
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll 1
      for (int kk = 0; kk < KT / 32; ++kk) {
        const int kb = kb0 + 32 * kk;
        const bool skip = kb > qw0 + 31 || (left >= 0 && kb + 31 < qw0 - left);
        if (!skip) masked(Kt, Vt, 32 * kk, kb);
      }
    }
  }
  __syncthreads();  // every wave is done with the K / V tiles: they become output slices
  static_assert(4 * store_slice_elems<HD>() <= 2 * KT * HD, "output slices fit the K tiles");
  store_rows<HD>(dqkv + ((long)b * Tn + qw0) * ld + h * HD, ld, min(32, Tn - qw0), dq, scale,
                 &Ks[0][0] + wave * store_slice_elems<HD>(), lane);
}

// Sequences whose packed qkv rows exceed what a 32-bit buffer offset reaches
// are rejected (T * 3 * H * hd * 2 bytes < 2 GiB).
inline bool fits_rsrc(int T, int H, int HD) { return (long)T * 3 * H * HD * 2 < 0x7fffffffL; }

template <int HD>
hipError_t launch_fwd(int B, int T, int H, int left, const void* qkv, void* out, float* lse,
                      hipStream_t s) {
  if (!fits_rsrc(T, H, HD)) return hipErrorInvalidValue;
  dim3 grid((unsigned)(B * H), (unsigned)cdiv(T, 128));
  float sl2 = LOG2E / sqrtf((float)HD);
  attn_fwd_mfma<HD><<<grid, 256, 0, s>>>((const bf16_t*)qkv, (bf16_t*)out, lse, T, H, left, sl2);
  return hipGetLastError();
}

template <int HD>
// dQ first: it also writes D and L2 (per query), which dK/dV then reads.
hipError_t launch_bwd(int B, int T, int H, int left, const void* qkv, const void* out,
                      const float* lse, const void* dout, float* D, float* L2, void* dqkv,
                      hipStream_t s) {
  if (!fits_rsrc(T, H, HD)) return hipErrorInvalidValue;
  dim3 grid((unsigned)(B * H), (unsigned)cdiv(T, 128));
  float sc = 1.f / sqrtf((float)HD);
  float sl2 = sc * LOG2E;
  attn_dq_mfma<HD><<<grid, 256, 0, s>>>((const bf16_t*)qkv, lse, (const bf16_t*)out,
                                        (const bf16_t*)dout, D, L2, (bf16_t*)dqkv, T, H, left,
                                        sc, sl2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_dkv_mfma<HD><<<grid, 256, 0, s>>>((const bf16_t*)qkv, L2, (const bf16_t*)dout, D,
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

hipError_t attention_scratch(long floats, float** out) {
  if (floats < 0 || floats > ATTN_SCRATCH_FLOATS) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::vector<float*> addr;  // per device, filled on the first call there
  std::lock_guard<std::mutex> lock(mu);
  if ((size_t)dev >= addr.size()) addr.resize((size_t)dev + 1, nullptr);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = (float*)p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t attention_bwd(int prec, int B, int T, int H, int hd, int left, const void* qkv,
                         const void* out, const float* lse, const void* dout, void* dqkv,
                         float* dvec, hipStream_t s) {
  if ((long)B * T * H == 0) return hipSuccess;
  if (!attention_supported(prec, hd)) return hipErrorInvalidValue;
  long rows = (long)B * T * H;
  if (prec == GPT_BF16) {
    float* L2 = dvec + rows;  // second half of the workspace
    if (hd == 32) return launch_bwd<32>(B, T, H, left, qkv, out, lse, dout, dvec, L2, dqkv, s);
    if (hd == 64) return launch_bwd<64>(B, T, H, left, qkv, out, lse, dout, dvec, L2, dqkv, s);
    return launch_bwd<128>(B, T, H, left, qkv, out, lse, dout, dvec, L2, dqkv, s);
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
