// Matrix products of the GPT step: C = op(A) . op(B)^T with fused epilogues.
//
// Every Linear layer of the model (nanoGPT README: model.py defines the GPT;
// nanochat "FLOPs-Berechnung im Detail": each matmul parameter
// costs 2 FLOPs forward and 4 backward) runs through here three times:
//   forward  y  = x W^T            A = x  [M,K]            B = W [N,K]
//   backward dx = dy W             A = dy [M,K]            B = W stored [K,N]
//   backward dW = dy^T x           A = dy stored [K,M]     B = x stored [K,N]
//
// bf16 path: CDNA4 MFMA (v_mfma_f32_32x32x16_bf16) with float accumulation.
// Output tiles of 256 x 256 (8 waves of 128 x 64, one workgroup per CU),
// 256 x 192 (8 waves of 64 x 96; N = 768 products) or 128 x 128 (4 waves of
// 64 x 64, two workgroups per CU).  K is staged through LDS in 64-deep slices,
// two stages, fetched straight from memory into LDS by buffer_load ... lds
// (no register staging): row-major tiles land with their 16-byte chunks XOR-
// swizzled per row, K-major tiles land untransposed and their MFMA fragments
// are read with the LDS transpose read (ds_read_b64_tr_b16).  An operand that
// takes GELU as it is read goes through registers instead (gemm_mfma_kernel).
// Long-K products (the weight gradients, K = B*T) are split over K into float
// partial tiles that a second kernel sums in a fixed order, so results are
// bitwise reproducible.
// fp32 path: a plain LDS-tiled FMA kernel (correctness path; small shapes).

#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <climits>
#include <cstdlib>
#include <type_traits>

namespace gpt {

namespace {

struct EpiArgs {
  int epi, tanh_form, M, N;
  const float* bias;
  const float* resid;
  void* out;
  long ldo;
  void* aux;
  long ldaux;
  float alpha, beta;           // AXPBY
  int batch;                   // > 1: grid z indexes the matrix of a batch
  long sa, sb, so, saux;       // byte strides between the matrices of a batch
};

template <typename ActT>
__device__ __forceinline__ void epilogue(const EpiArgs& e, int m, int n, float acc) {
  if (m >= e.M || n >= e.N) return;
  long o = (long)m * e.ldo + n;
  switch (e.epi) {
    case GPT_EPI_STORE:
      if (e.bias) acc += e.bias[n];
      Act<ActT>::store((ActT*)e.out, o, acc);
      break;
    case GPT_EPI_RESIDUAL:
      if (e.bias) acc += e.bias[n];
      ((float*)e.out)[o] = e.resid[o] + acc;
      break;
    case GPT_EPI_GELU:
      if (e.bias) acc += e.bias[n];
      Act<ActT>::store((ActT*)e.out, o, acc);
      if (e.aux) {
        // GELU of the stored (rounded) pre-activation, as a recompute would see it.
        float u = Act<ActT>::load((const ActT*)e.out, o);
        Act<ActT>::store((ActT*)e.aux, (long)m * e.ldaux + n, gelu_f(u, e.tanh_form));
      }
      break;
    case GPT_EPI_DGELU: {
      float u = Act<ActT>::load((const ActT*)e.aux, (long)m * e.ldaux + n);
      Act<ActT>::store((ActT*)e.out, o, acc * gelu_grad_f(u, e.tanh_form));
      break;
    }
    case GPT_EPI_GELU_PAIR: {
      if (e.bias) acc += e.bias[n];
      ActT r;  // the pre-activation rounded to the activation type
      Act<ActT>::store(&r, 0, acc);
      const float u = Act<ActT>::load(&r, 0);
      Act<ActT>::store((ActT*)e.out, o, gelu_grad_f(u, e.tanh_form));
      Act<ActT>::store((ActT*)e.aux, (long)m * e.ldaux + n, gelu_f(u, e.tanh_form));
      break;
    }
    case GPT_EPI_MUL:
      Act<ActT>::store((ActT*)e.out, o,
                       acc * Act<ActT>::load((const ActT*)e.aux, (long)m * e.ldaux + n));
      break;
    case GPT_EPI_AXPBY:
      Act<ActT>::store((ActT*)e.out, o,
                       e.alpha * acc +
                           e.beta * Act<ActT>::load((const ActT*)e.aux, (long)m * e.ldaux + n));
      break;
    case GPT_EPI_F32:
      ((float*)e.out)[o] = acc;
      break;
    case GPT_EPI_F32_ACCUM:
      ((float*)e.out)[o] += acc;
      break;
  }
}

struct OpArgs {
  const void* X;
  long ld;
  int trans, rows, kvalid, gelu;
};

// Matrix z of a batched product: operand and output bases moved by the
// batch strides.
__device__ __forceinline__ void batch_select(int z, OpArgs& a, OpArgs& b, EpiArgs& e) {
  a.X = (const char*)a.X + z * e.sa;
  b.X = (const char*)b.X + z * e.sb;
  e.out = (char*)e.out + z * e.so;
  if (e.aux) e.aux = (char*)e.aux + z * e.saux;
}

// ----------------------------------------------------------------------------
// fp32 / generic path: 64x64 tile, 16x16 threads, 4x4 outputs per thread.
// ----------------------------------------------------------------------------
template <typename InT>
__device__ __forceinline__ float load_elem(const OpArgs& a, int r, int k, int tanh_form) {
  if (r >= a.rows || k >= a.kvalid) return 0.f;
  long off = a.trans ? (long)k * a.ld + r : (long)r * a.ld + k;
  float v = Act<InT>::load((const InT*)a.X, off);
  if (a.gelu) v = gelu_f(v, tanh_form);
  return v;
}

template <typename InT, typename ActT>
__global__ void __launch_bounds__(256) gemm_simt_kernel(OpArgs A, OpArgs B, int K, EpiArgs e) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  if (e.batch > 1) batch_select(blockIdx.z, A, B, e);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = threadIdx.x; i < 64 * 16; i += 256) {
      int r = i % 64, k = i / 64;
      As[k][r] = load_elem<InT>(A, m0 + r, k0 + k, e.tanh_form);
      Bs[k][r] = load_elem<InT>(B, n0 + r, k0 + k, e.tanh_form);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) epilogue<ActT>(e, m0 + ty * 4 + i, n0 + tx * 4 + j, acc[i][j]);
}

// ----------------------------------------------------------------------------
// bf16 MFMA path.
// ----------------------------------------------------------------------------
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int EPI_PARTIAL = 100;  // split-K: raw float partial tile

// LDS operand tile: [128 rows][BK] bf16, 128 bytes per row, its eight 16-byte
// chunks XOR-swizzled by f(row) = (row & 7) ^ ((row >> 3) & 1).  With 64 banks
// two consecutive rows share a bank line, so a 16-lane group of a fragment
// read (rows r..r+15, one logical chunk) needs distinct chunks among the rows
// of equal parity; f gives that (and distinct chunks for any 8 consecutive
// rows, the 32-bank case).
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 3);
}

// GELU of a packed bf16 pair (bf16 path only: fast form).
__device__ __forceinline__ uint32_t gelu2(uint32_t w, int tanh_form) {
  return pack_bf2(gelu_fast(bf_lo(w), tanh_form), gelu_fast(bf_hi(w), tanh_form));
}

// Global -> registers for one BK-slice of a 128-row operand tile: 4 vectors
// of 8 bf16 per thread, full 16-byte coalesced loads in both layouts.
//  row-major (K contiguous): vector (row, chunk) = (v / 8, v % 8), v = t + 256 i.
//  K-major (rows contiguous): vector (k, rchunk) = (v / 16, v % 16); the tile
//    lands in LDS untransposed as [BK][128] and the MFMA fragments are read
//    with the LDS transpose read (see tr_frag).
struct Stage { u32x4 v[4]; };

template <int TRANS, bool GELU>
__device__ __forceinline__ void stage_load(const OpArgs& a, int r0, int k0, int tanh_form,
                                           Stage& st) {
  const int t = threadIdx.x;
  const bf16_t* X = (const bf16_t*)a.X;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int vix = t + 256 * i;
    u32x4 val = {0, 0, 0, 0};
    if constexpr (TRANS == 0) {
      const int r = r0 + (vix >> 3), k = k0 + (vix & 7) * 8;
      if (r < a.rows && k < a.kvalid) val = *(const u32x4*)(X + (long)r * a.ld + k);
    } else {
      const int k = k0 + (vix >> 4), r = r0 + (vix & 15) * 8;
      if (r < a.rows && k < a.kvalid) val = *(const u32x4*)(X + (long)k * a.ld + r);
    }
    if (GELU) val = u32x4{gelu2(val.x, tanh_form), gelu2(val.y, tanh_form),
                          gelu2(val.z, tanh_form), gelu2(val.w, tanh_form)};
    st.v[i] = val;
  }
}

// K-major LDS tile [BK][128]: 256-byte rows whose four 64-byte granules are
// XOR-swizzled by (k & 3), so the 4 K-rows a transpose read touches at once
// sit in different banks.
__device__ __forceinline__ int lds_off_t(int k, int r) { return k * 128 + (r ^ ((k & 3) << 5)); }

template <int TRANS>
__device__ __forceinline__ void stage_store(const Stage& st, bf16_t* lds) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int vix = t + 256 * i;
    if constexpr (TRANS == 0)
      *(u32x4*)(lds + lds_off(vix >> 3, vix & 7)) = st.v[i];
    else
      *(u32x4*)(lds + lds_off_t(vix >> 4, (vix & 15) * 8)) = st.v[i];
  }
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// MFMA 32x32x16 operand fragment (row r0 + lane % 32, k-slots 16 ks + 8 (lane / 32)
// + 0..7) from a K-major tile with two LDS transpose reads.  Within each group
// of 16 lanes, source lane s = a + 4 b supplies the 4 values at (k = kb + b,
// rows 4a .. 4a + 3); lane j of the group then receives rows j, k = kb .. kb + 3.
__device__ __forceinline__ bf16x8 tr_frag(const bf16_t* lds, int r0, int ks, int lane) {
  const int s = lane & 15, grp = lane >> 4;
  const int r = r0 + 16 * (grp & 1) + 4 * (s & 3);
  const int kb = ks * 16 + 8 * (grp >> 1) + (s >> 2);
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + lds_off_t(kb, r)));
  v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + lds_off_t(kb + 4, r)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return *(bf16x8*)&v;
}

template <int TRANS>
__device__ __forceinline__ bf16x8 frag(const bf16_t* lds, int r0, int ks, int lane) {
  if constexpr (TRANS == 0)
    return *(const bf16x8*)(lds + lds_off(r0 + (lane & 31), ks * 2 + (lane >> 5)));
  else
    return tr_frag(lds, r0, ks, lane);
}

// Epilogue on 8 consecutive columns n..n+7 of row m (n + 8 <= N, rows 16-byte aligned).
// 16-byte output stores.  The non-temporal form (plain STORE / GELU outputs:
// the vocabulary projection's 1.6 GB of logits above all) does not allocate
// in the L2, so the operand panels keep the cache; measured neutral to worse
// for the epilogues that also read an auxiliary input, which keep plain stores.
__device__ __forceinline__ void st16nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, (u32x4*)p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }

// The MUL epilogue (out = acc * aux) with its 8 auxiliary values already loaded.
__device__ __forceinline__ void mul8_store(const EpiArgs& e, int m, int n, float4 v0, float4 v1,
                                           u32x4 a) {
  st16((bf16_t*)e.out + (long)m * e.ldo + n,
       u32x4{pack_bf2(v0.x * bf_lo(a.x), v0.y * bf_hi(a.x)),
             pack_bf2(v0.z * bf_lo(a.y), v0.w * bf_hi(a.y)),
             pack_bf2(v1.x * bf_lo(a.z), v1.y * bf_hi(a.z)),
             pack_bf2(v1.z * bf_lo(a.w), v1.w * bf_hi(a.w))});
}

template <int EPI>
__device__ __forceinline__ void epilogue8(const EpiArgs& e, float* partial, int m, int n,
                                          float4 v0, float4 v1) {
  const long o = (long)m * e.ldo + n;
  float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  if constexpr (EPI == EPI_PARTIAL) {
    float* p = partial + (long)m * e.N + n;  // this split's partial tile
    *(float4*)p = v0;
    *(float4*)(p + 4) = v1;
    return;
  }
  if constexpr (EPI == GPT_EPI_STORE || EPI == GPT_EPI_RESIDUAL || EPI == GPT_EPI_GELU) {
    if (e.bias) {
      float4 b0 = *(const float4*)(e.bias + n), b1 = *(const float4*)(e.bias + n + 4);
      x[0] += b0.x; x[1] += b0.y; x[2] += b0.z; x[3] += b0.w;
      x[4] += b1.x; x[5] += b1.y; x[6] += b1.z; x[7] += b1.w;
    }
  }
  if constexpr (EPI == GPT_EPI_STORE || EPI == GPT_EPI_GELU) {
    u32x4 w{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]),
            pack_bf2(x[6], x[7])};
    st16nt((bf16_t*)e.out + o, w);
    if constexpr (EPI == GPT_EPI_GELU) {
      if (e.aux) {
        // GELU of the stored (rounded) pre-activation, as a recompute would see it.
        u32x4 g{gelu2(w.x, e.tanh_form), gelu2(w.y, e.tanh_form), gelu2(w.z, e.tanh_form),
                gelu2(w.w, e.tanh_form)};
        st16nt((bf16_t*)e.aux + (long)m * e.ldaux + n, g);
      }
    }
  } else if constexpr (EPI == GPT_EPI_DGELU) {
    u32x4 u = *(const u32x4*)((const bf16_t*)e.aux + (long)m * e.ldaux + n);
    const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] *= gelu_grad_fast(bf_lo(uw[i]), e.tanh_form);
      x[2 * i + 1] *= gelu_grad_fast(bf_hi(uw[i]), e.tanh_form);
    }
    st16((bf16_t*)e.out + o, u32x4{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]),
                                           pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7])});
  } else if constexpr (EPI == GPT_EPI_MUL) {
    const u32x4 a = *(const u32x4*)((const bf16_t*)e.aux + (long)m * e.ldaux + n);
    st16((bf16_t*)e.out + o, u32x4{
        pack_bf2(x[0] * bf_lo(a.x), x[1] * bf_hi(a.x)), pack_bf2(x[2] * bf_lo(a.y), x[3] * bf_hi(a.y)),
        pack_bf2(x[4] * bf_lo(a.z), x[5] * bf_hi(a.z)), pack_bf2(x[6] * bf_lo(a.w), x[7] * bf_hi(a.w))});
  } else if constexpr (EPI == GPT_EPI_AXPBY) {
    const u32x4 a = *(const u32x4*)((const bf16_t*)e.aux + (long)m * e.ldaux + n);
    const float al = e.alpha, be = e.beta;
    st16((bf16_t*)e.out + o, u32x4{
        pack_bf2(al * x[0] + be * bf_lo(a.x), al * x[1] + be * bf_hi(a.x)),
        pack_bf2(al * x[2] + be * bf_lo(a.y), al * x[3] + be * bf_hi(a.y)),
        pack_bf2(al * x[4] + be * bf_lo(a.z), al * x[5] + be * bf_hi(a.z)),
        pack_bf2(al * x[6] + be * bf_lo(a.w), al * x[7] + be * bf_hi(a.w))});
  } else if constexpr (EPI == GPT_EPI_GELU_PAIR) {
    if (e.bias) {
      float4 b0 = *(const float4*)(e.bias + n), b1 = *(const float4*)(e.bias + n + 4);
      x[0] += b0.x; x[1] += b0.y; x[2] += b0.z; x[3] += b0.w;
      x[4] += b1.x; x[5] += b1.y; x[6] += b1.z; x[7] += b1.w;
    }
    const u32x4 w{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]),
                  pack_bf2(x[6], x[7])};  // u rounded to bf16
    float g[8], gp[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gelu_pair_fast(bf_lo(w[i]), e.tanh_form, g[2 * i], gp[2 * i]);
      gelu_pair_fast(bf_hi(w[i]), e.tanh_form, g[2 * i + 1], gp[2 * i + 1]);
    }
    // GELU'(u) is read only by the backward pass: streamed past the caches
    // (GELU(u), the next product's operand, is stored normally).
    st16nt((bf16_t*)e.out + o, u32x4{pack_bf2(gp[0], gp[1]), pack_bf2(gp[2], gp[3]),
                                           pack_bf2(gp[4], gp[5]), pack_bf2(gp[6], gp[7])});
    st16((bf16_t*)e.aux + (long)m * e.ldaux + n, u32x4{
        pack_bf2(g[0], g[1]), pack_bf2(g[2], g[3]), pack_bf2(g[4], g[5]), pack_bf2(g[6], g[7])});
  } else if constexpr (EPI == GPT_EPI_RESIDUAL) {
    float4 r0 = *(const float4*)(e.resid + o), r1 = *(const float4*)(e.resid + o + 4);
    *(float4*)((float*)e.out + o) = make_float4(r0.x + x[0], r0.y + x[1], r0.z + x[2], r0.w + x[3]);
    *(float4*)((float*)e.out + o + 4) =
        make_float4(r1.x + x[4], r1.y + x[5], r1.z + x[6], r1.w + x[7]);
  } else if constexpr (EPI == GPT_EPI_F32) {
    *(float4*)((float*)e.out + o) = v0;
    *(float4*)((float*)e.out + o + 4) = v1;
  } else if constexpr (EPI == GPT_EPI_F32_ACCUM) {
    float4* p = (float4*)((float*)e.out + o);
    float4 a0 = p[0], a1 = p[1];
    p[0] = make_float4(a0.x + x[0], a0.y + x[1], a0.z + x[2], a0.w + x[3]);
    p[1] = make_float4(a1.x + x[4], a1.y + x[5], a1.z + x[6], a1.w + x[7]);
  }
}

template <int AT, int BT, int EPI, bool GA, bool GB>
__global__ void __launch_bounds__(256, 2) gemm_mfma_kernel(OpArgs A, OpArgs B, int K, int kchunk,
                                                           EpiArgs e, float* partial) {
  // Two stages of A and B tiles (4 x 16 KB); reused as the 128 x 128 float
  // output tile by the epilogue.
  __shared__ __attribute__((aligned(16))) char smem[4 * BM * BK * 2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  int zs = blockIdx.z;  // K split, or the matrix of a batch
  if (e.batch > 1) {
    batch_select(zs, A, B, e);
    zs = 0;
  }
  const int kbeg = zs * kchunk;
  if (EPI == EPI_PARTIAL) partial += (long)zs * e.M * e.N;
  const int kend = min(K, kbeg + kchunk);
  const int nk = (kend - kbeg + BK - 1) / BK;
  // Stage s: A tile at smem + s * 32 KB, B tile 16 KB after it.
  auto a_tile = [&](int st) { return (bf16_t*)(smem + st * 2 * BM * BK * 2); };
  auto b_tile = [&](int st) { return (bf16_t*)(smem + st * 2 * BM * BK * 2 + BM * BK * 2); };

  f32x16 acc00 = {}, acc01 = {}, acc10 = {}, acc11 = {};

  // The K range of this split is [kbeg, kend); clamp operand validity to it.
  OpArgs a = A, b = B;
  a.kvalid = min(a.kvalid, kend);
  b.kvalid = min(b.kvalid, kend);

  Stage sa, sb;
  stage_load<AT, GA>(a, m0, kbeg, e.tanh_form, sa);
  stage_load<BT, GB>(b, n0, kbeg, e.tanh_form, sb);
  stage_store<AT>(sa, a_tile(0));
  stage_store<BT>(sb, b_tile(0));
  __syncthreads();

  const int frow = lane & 31, fg = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      stage_load<AT, GA>(a, m0, kbeg + (kt + 1) * BK, e.tanh_form, sa);
      stage_load<BT, GB>(b, n0, kbeg + (kt + 1) * BK, e.tanh_form, sb);
    }
    const bf16_t* as = a_tile(cur);
    const bf16_t* bs = b_tile(cur);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const bf16x8 a0 = frag<AT>(as, wm * 64, ks, lane);
      const bf16x8 a1 = frag<AT>(as, wm * 64 + 32, ks, lane);
      const bf16x8 b0 = frag<BT>(bs, wn * 64, ks, lane);
      const bf16x8 b1 = frag<BT>(bs, wn * 64 + 32, ks, lane);
      acc00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc00, 0, 0, 0);
      acc01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc01, 0, 0, 0);
      acc10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc10, 0, 0, 0);
      acc11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc11, 0, 0, 0);
    }
    if (more) {
      stage_store<AT>(sa, a_tile(cur ^ 1));
      stage_store<BT>(sb, b_tile(cur ^ 1));
    }
    __syncthreads();
  }

  // Accumulators -> LDS float tile [128][128].  32x32 block layout:
  // column = lane % 32, row = 8 * (r / 4) + 4 * (lane / 32) + r % 4.
  float* Cs = (float*)smem;
  {
    const int rb = wm * 64 + 4 * fg, cb = wn * 64 + frow;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rb + 8 * (r >> 2) + (r & 3);
      Cs[row * BN + cb] = acc00[r];
      Cs[row * BN + cb + 32] = acc01[r];
      Cs[(row + 32) * BN + cb] = acc10[r];
      Cs[(row + 32) * BN + cb + 32] = acc11[r];
    }
  }
  __syncthreads();
  // Coalesced epilogue: 16 threads per row, 8 consecutive columns each.
  const int cg = threadIdx.x & 15;
  const int n = n0 + cg * 8;
  if (n >= e.N) return;
  for (int pass = 0; pass < BM / 16; ++pass) {
    const int row = pass * 16 + (threadIdx.x >> 4);
    const int m = m0 + row;
    if (m >= e.M) break;
    const float4 v0 = *(const float4*)(Cs + row * BN + cg * 8);
    const float4 v1 = *(const float4*)(Cs + row * BN + cg * 8 + 4);
    epilogue8<EPI>(e, partial, m, n, v0, v1);
  }
}

template <typename ActT>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* partial, int S, EpiArgs e) {
  long total = (long)e.M * e.N;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    float s = 0.f;
    for (int z = 0; z < S; ++z) s += partial[(long)z * total + i];
    epilogue<ActT>(e, (int)(i / e.N), (int)(i % e.N), s);
  }
}

// Split-K reduction, 8 consecutive columns per thread (N % 8 == 0, 16-byte
// aligned rows): partials summed in z order, then the vector epilogue.
template <int EPI>
__global__ void __launch_bounds__(256) splitk_reduce8_kernel(const float* __restrict__ partial,
                                                             int S, EpiArgs e) {
  const long per_row = e.N / 8, total = (long)e.M * per_row;
  const long plane = (long)e.M * e.N;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    const int m = (int)(i / per_row), n = (int)(i % per_row) * 8;
    const float* p = partial + (long)m * e.N + n;
    float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    for (int z = 1; z < S; ++z) {
      const float4 c = *(const float4*)(p + z * plane), d = *(const float4*)(p + z * plane + 4);
      a.x += c.x; a.y += c.y; a.z += c.z; a.w += c.w;
      b.x += d.x; b.y += d.y; b.z += d.z; b.w += d.w;
    }
    epilogue8<EPI>(e, nullptr, m, n, a, b);
  }
}

typedef void (*MfmaKernel)(OpArgs, OpArgs, int, int, EpiArgs, float*);

// The specialisations the training step uses; anything else takes the
// generic kernel.  Key: (a_trans, b_trans, epilogue, a_gelu, b_gelu).
MfmaKernel mfma_kernel_for(int at, int bt, int epi, int ga, int gb) {
#define K_(AT, BT, EP, GA, GB)                                        \
  if (at == AT && bt == BT && epi == EP && ga == GA && gb == GB)      \
    return gemm_mfma_kernel<AT, BT, EP, GA, GB>;
  K_(0, 0, GPT_EPI_STORE, 0, 0)
  K_(0, 0, GPT_EPI_RESIDUAL, 0, 0)
  K_(0, 0, GPT_EPI_RESIDUAL, 1, 0)
  K_(0, 0, GPT_EPI_GELU, 0, 0)
  K_(0, 0, GPT_EPI_DGELU, 0, 0)
  K_(0, 0, GPT_EPI_GELU_PAIR, 0, 0)
  K_(0, 0, GPT_EPI_F32, 0, 0)
  K_(0, 0, GPT_EPI_F32_ACCUM, 0, 0)
  K_(0, 1, GPT_EPI_STORE, 0, 0)
  K_(0, 1, GPT_EPI_DGELU, 0, 0)
  K_(0, 1, GPT_EPI_MUL, 0, 0)
  K_(0, 1, GPT_EPI_F32, 0, 0)
  K_(0, 0, GPT_EPI_AXPBY, 0, 0)
  K_(0, 0, EPI_PARTIAL, 0, 0)
  K_(0, 1, GPT_EPI_AXPBY, 0, 0)
  K_(1, 1, GPT_EPI_STORE, 0, 0)
  K_(1, 1, GPT_EPI_F32, 0, 0)
  K_(1, 1, GPT_EPI_F32_ACCUM, 0, 0)
  K_(1, 1, EPI_PARTIAL, 0, 0)
  K_(1, 1, GPT_EPI_F32, 0, 1)
  K_(1, 1, GPT_EPI_F32_ACCUM, 0, 1)
  K_(1, 1, EPI_PARTIAL, 0, 1)
#undef K_
  return nullptr;
}

// Workgroups are dealt round-robin over the 8 XCDs (each with its own 4 MB
// L2).  Renumber them so every XCD owns a contiguous run of tile ids (all the
// tiles of a K split stay on one XCD), and order each split's tiles in groups
// of TILE_GROUP tile-rows walked column by column: the workgroups resident on
// an XCD at one time then share a few A row panels and B column panels, so
// each K slice of an operand is fetched into the L2 once and read there by
// every tile that needs it.
constexpr int TILE_GROUP = 8;
__device__ __forceinline__ void xcd_tile(int& tx, int& ty, int& tz) {
  const int nx = gridDim.x, ny = gridDim.y;
  const int per_z = nx * ny, total = per_z * gridDim.z;
  const int L = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  int id = L;
  if ((total & 7) == 0) id = (L & 7) * (total >> 3) + (L >> 3);
  tz = id / per_z;
  const int r = id - tz * per_z;
  const int g = r / (TILE_GROUP * nx);
  const int rows = min(TILE_GROUP, ny - g * TILE_GROUP);
  const int w = r - g * TILE_GROUP * nx;
  tx = w / rows;
  ty = g * TILE_GROUP + w % rows;
}

// ----------------------------------------------------------------------------
// bf16 MFMA, 128 x 128 tile, operands fetched straight into LDS with buffer
// loads (buffer_load_dwordx4 ... lds): no register staging and no LDS store
// instructions; the loads of tile k+1 run while tile k is multiplied.  One
// wave instruction fills a contiguous 1 KB LDS block (lane l -> bytes 16 l),
// so the XOR swizzle of the LDS layouts is applied to the SOURCE address each
// lane picks.  Lanes outside the valid rows / K range get an offset past the
// buffer's range and read zeros.
// ----------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
  const int n = bytes > 0x7fffffffL ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, n, 0x00020000);
}

// One 16-byte direct-to-LDS load per lane into the wave's 1 KB block at
// `lds` (lane l -> bytes 16 l).  With ASM the load is issued from inline asm
// (M0 = the block's LDS address, set in the same statement; no register
// result): the compiler's wait insertion then does not treat it as a pending
// write of the LDS the fragment reads of the current stage use.  Without it,
// the compiler places a vmcnt(0) right after the next stage's loads wherever
// fragments are read with the LDS transpose builtin, so those loads never
// overlap the MFMAs.  Kernels using ASM order their loads themselves: every
// stage ends with vmcnt(0) and a barrier before its buffer is read or refilled.
template <bool ASM>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, bf16_t* lds, unsigned off) {
  if constexpr (ASM) {
    const unsigned m0v = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0v), "v"(off), "s"(rs)
                 : "memory", "m0");
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, off, 0, 0, 0);
  }
}

// Issue this wave's 4 loads of one 128 x BK operand tile into `lds`.
template <int TRANS, bool ASM = false>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, const OpArgs& a, int r0,
                                         int k0, bf16_t* lds, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = wave * 4 + i;  // 1 KB block of the 16 KB tile
    int r, k;
    if constexpr (TRANS == 0) {  // [128 rows][64 k]: block = 8 rows x 8 chunks
      const int row = blk * 8 + (lane >> 3), phys = lane & 7;
      const int chunk = phys ^ (row & 7) ^ ((row >> 3) & 1);
      r = r0 + row;
      k = k0 + chunk * 8;
    } else {  // [64 k][128 rows]: block = 4 k-rows x 16 chunks
      const int kk = blk * 4 + (lane >> 4), phys = lane & 15;
      const int chunk = phys ^ ((kk & 3) << 2);
      k = k0 + kk;
      r = r0 + chunk * 8;
    }
    const bool ok = r < a.rows && k < a.kvalid;
    const long e = TRANS ? (long)k * a.ld + r : (long)r * a.ld + k;
    const unsigned off = ok ? (unsigned)(e * 2) : 0x80000000u;
    dma16<ASM>(rs, lds + blk * 512, off);
  }
}

// Scheduling groups for one 16-deep step of NM MFMAs (4 or 8) with the NDS
// LDS reads of the next step spread evenly after them.
template <int N> __device__ __forceinline__ void sched_ds() {
  if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(0x100, N, 0);
}
template <int NM, int NDS, int Q = 0> __device__ __forceinline__ void sched_mfma_ds() {
  if constexpr (Q < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    sched_ds<NDS / NM + (Q < NDS % NM ? 1 : 0)>();
    sched_mfma_ds<NM, NDS, Q + 1>();
  }
}

template <int AT, int BT, int EPI>
__global__ void __launch_bounds__(256, 2) gemm_dma_kernel(OpArgs A, OpArgs B, int K, int kchunk,
                                                          EpiArgs e, float* partial) {
  // One 64 KB block: two stages of A and B tiles, later the float output tile.
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (BM + BN) * BK];
  bf16_t* const sA0 = smem;
  bf16_t* const sB0 = smem + BM * BK;
  bf16_t* const sA1 = smem + (BM + BN) * BK;
  bf16_t* const sB1 = smem + (2 * BM + BN) * BK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tx, ty, tz;
  xcd_tile(tx, ty, tz);
  if (e.batch > 1) {  // tz indexes the matrix of a batch (never split over K)
    batch_select(tz, A, B, e);
    tz = 0;
  }
  const int m0 = ty * BM, n0 = tx * BN;
  const int kbeg = tz * kchunk;
  if (EPI == EPI_PARTIAL) partial += (long)tz * e.M * e.N;
  const int kend = min(K, kbeg + kchunk);
  const int nk = (kend - kbeg + BK - 1) / BK;

  OpArgs a = A, b = B;
  a.kvalid = min(a.kvalid, kend);
  b.kvalid = min(b.kvalid, kend);
  const long a_extent = AT ? (long)a.kvalid * a.ld : (long)a.rows * a.ld;
  const long b_extent = BT ? (long)b.kvalid * b.ld : (long)b.rows * b.ld;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.X, a_extent * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(b.X, b_extent * 2);

  f32x16 acc00 = {}, acc01 = {}, acc10 = {}, acc11 = {};

  dma_tile<AT, (AT || BT)>(ra, a, m0, kbeg, sA0, wave, lane);
  dma_tile<BT, (AT || BT)>(rb, b, n0, kbeg, sB0, wave, lane);
  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's loads of tile kt landed
    __syncthreads();                     // ... and every other wave's
    const bool odd = kt & 1;
    if (kt + 1 < nk) {
      const int k1 = kbeg + (kt + 1) * BK;
      dma_tile<AT, (AT || BT)>(ra, a, m0, k1, odd ? sA0 : sA1, wave, lane);
      dma_tile<BT, (AT || BT)>(rb, b, n0, k1, odd ? sB0 : sB1, wave, lane);
    }
    const bf16_t* as = odd ? sA1 : sA0;
    const bf16_t* bs = odd ? sB1 : sB0;
    // Fragments double-buffered across the 16-deep steps (see the 8-wave kernel).
    constexpr int NDS = (AT ? 4 : 2) + (BT ? 4 : 2);
    bf16x8 fa[2][2], fb[2][2];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      fa[0][h] = frag<AT>(as, wm * 64 + 32 * h, 0, lane);
      fb[0][h] = frag<BT>(bs, wn * 64 + 32 * h, 0, lane);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          fa[cur ^ 1][h] = frag<AT>(as, wm * 64 + 32 * h, ks + 1, lane);
          fb[cur ^ 1][h] = frag<BT>(bs, wn * 64 + 32 * h, ks + 1, lane);
        }
      }
      acc00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][0], fb[cur][0], acc00, 0, 0, 0);
      acc01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][0], fb[cur][1], acc01, 0, 0, 0);
      acc10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][1], fb[cur][0], acc10, 0, 0, 0);
      acc11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][1], fb[cur][1], acc11, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) sched_mfma_ds<4, NDS>();
      else __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(0x3f70);
  __syncthreads();

  // Accumulators -> LDS float tile [128][128] (the whole 64 KB block).
  float* Cs = (float*)smem;
  {
    const int frow = lane & 31, fg = lane >> 5;
    const int rb = wm * 64 + 4 * fg, cb = wn * 64 + frow;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rb + 8 * (r >> 2) + (r & 3);
      Cs[row * BN + cb] = acc00[r];
      Cs[row * BN + cb + 32] = acc01[r];
      Cs[(row + 32) * BN + cb] = acc10[r];
      Cs[(row + 32) * BN + cb + 32] = acc11[r];
    }
  }
  __syncthreads();
  const int cg = threadIdx.x & 15;
  const int n = n0 + cg * 8;
  if (n >= e.N) return;
  for (int pass = 0; pass < BM / 16; ++pass) {
    const int row = pass * 16 + (threadIdx.x >> 4);
    const int m = m0 + row;
    if (m >= e.M) break;
    const float4 v0 = *(const float4*)(Cs + row * BN + cg * 8);
    const float4 v1 = *(const float4*)(Cs + row * BN + cg * 8 + 4);
    epilogue8<EPI>(e, partial, m, n, v0, v1);
  }
}

MfmaKernel dma_kernel_for(int at, int bt, int epi, int ga, int gb) {
  if (ga || gb) return nullptr;
#define K_(AT, BT, EP) \
  if (at == AT && bt == BT && epi == EP) return gemm_dma_kernel<AT, BT, EP>;
  K_(0, 0, GPT_EPI_STORE)
  K_(0, 0, GPT_EPI_RESIDUAL)
  K_(0, 0, GPT_EPI_GELU)
  K_(0, 0, GPT_EPI_DGELU)
  K_(0, 0, GPT_EPI_GELU_PAIR)
  K_(0, 0, GPT_EPI_F32)
  K_(0, 0, GPT_EPI_F32_ACCUM)
  K_(0, 1, GPT_EPI_STORE)
  K_(0, 1, GPT_EPI_DGELU)
  K_(0, 1, GPT_EPI_MUL)
  K_(0, 1, GPT_EPI_F32)
  K_(0, 1, EPI_PARTIAL)
  K_(0, 0, GPT_EPI_AXPBY)
  K_(0, 0, EPI_PARTIAL)
  K_(0, 1, GPT_EPI_AXPBY)
  K_(1, 1, GPT_EPI_STORE)
  K_(1, 1, GPT_EPI_F32)
  K_(1, 1, GPT_EPI_F32_ACCUM)
  K_(1, 1, EPI_PARTIAL)
#undef K_
  return nullptr;
}

// ----------------------------------------------------------------------------
// bf16 MFMA, large tiles (256 rows): LDS layouts and fragment reads shared by
// the 256 x 256 and 256 x 192 kernels below.
// ----------------------------------------------------------------------------
constexpr int BIG = 256;

__device__ __forceinline__ int big_off(int row, int chunk) {  // row-major tile [256][BK]
  return row * BK + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 3);
}
__device__ __forceinline__ int big_off_t(int k, int r) {  // K-major tile [BK][256]
  return k * BIG + (r ^ ((k & 3) << 5));
}

template <int TRANS>
__device__ __forceinline__ bf16x8 big_frag(const bf16_t* lds, int r0, int ks, int lane) {
  if constexpr (TRANS == 0) {
    return *(const bf16x8*)(lds + big_off(r0 + (lane & 31), ks * 2 + (lane >> 5)));
  } else {
    const int s = lane & 15, grp = lane >> 4;
    const int r = r0 + 16 * (grp & 1) + 4 * (s & 3);
    const int kb = ks * 16 + 8 * (grp >> 1) + (s >> 2);
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + big_off_t(kb, r)));
    v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + big_off_t(kb + 4, r)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return *(bf16x8*)&v;
  }
}

// ----------------------------------------------------------------------------
// bf16 MFMA, 256 x 256 tile with 8 waves (2 along M x 4 along N, 128 x 64
// each): two waves per SIMD, so one wave's LDS reads and load waits hide
// behind the other's MFMAs, at 1.5x the LDS reads per FLOP of the 4-wave
// layout.  BK = 64, two 64 KB LDS stages filled by direct buffer loads (four
// 1 KB blocks per wave and operand per stage); the epilogue stages each
// wave's 32-row slices through LDS for 16-byte vector stores.
// ----------------------------------------------------------------------------
template <int TRANS, bool ASM = false>
__device__ __forceinline__ void dma_tile256_w8(__amdgpu_buffer_rsrc_t rs, const OpArgs& a, int r0,
                                               int k0, bf16_t* lds, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = wave * 4 + i;  // 1 KB block of the 32 KB tile
    int r, k;
    if constexpr (TRANS == 0) {  // block = 8 rows x 8 chunks
      const int row = blk * 8 + (lane >> 3), phys = lane & 7;
      const int chunk = phys ^ (row & 7) ^ ((row >> 3) & 1);
      r = r0 + row;
      k = k0 + chunk * 8;
    } else {  // block = 2 k-rows x 32 chunks
      const int kk = blk * 2 + (lane >> 5), phys = lane & 31;
      const int chunk = phys ^ ((kk & 3) << 2);
      k = k0 + kk;
      r = r0 + chunk * 8;
    }
    const bool ok = r < a.rows && k < a.kvalid;
    const long e = TRANS ? (long)k * a.ld + r : (long)r * a.ld + k;
    const unsigned off = ok ? (unsigned)(e * 2) : 0x80000000u;
    dma16<ASM>(rs, lds + blk * 512, off);
  }
}

// The same loads for a k-tile that lies wholly inside both operands' K range:
// the per-lane source offsets (bytes, relative to the tile's first K) are
// computed once per tile by dma_plan256_w8, and the k-tile's own K offset goes
// in the instruction's scalar offset, so a load costs no vector arithmetic.
// Rows past the operand keep an offset beyond the buffer's range (zeros).
template <int TRANS>
__device__ __forceinline__ void dma_plan256_w8(const OpArgs& a, int r0, int kbeg, int wave,
                                               int lane, unsigned (&voff)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = wave * 4 + i;
    int r, k;
    if constexpr (TRANS == 0) {
      const int row = blk * 8 + (lane >> 3), phys = lane & 7;
      const int chunk = phys ^ (row & 7) ^ ((row >> 3) & 1);
      r = r0 + row;
      k = kbeg + chunk * 8;
    } else {
      const int kk = blk * 2 + (lane >> 5), phys = lane & 31;
      const int chunk = phys ^ ((kk & 3) << 2);
      k = kbeg + kk;
      r = r0 + chunk * 8;
    }
    const long e = TRANS ? (long)k * a.ld + r : (long)r * a.ld + k;
    voff[i] = r < a.rows ? (unsigned)(e * 2) : 0x80000000u;
  }
}
__device__ __forceinline__ void dma_fast256_w8(__amdgpu_buffer_rsrc_t rs, const unsigned (&voff)[4],
                                               unsigned soff, bf16_t* lds, int wave_s) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned m0v = (unsigned)(uintptr_t)(lds + (wave_s * 4 + i) * 512);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0v), "v"(voff[i]), "s"(rs), "s"(soff)
                 : "memory", "m0");
  }
}

// One 256 x 256 output tile (tx, ty) over the K range of split tz; `smem` is
// the kernel's 128 KB LDS block (two stages of A and B tiles, later the
// epilogue slices).
// CSUM (K-major A only): when `csum` is set, the tile's column sums of A over
// its K range (sum_k A(m, k) for its 256 rows m: a Linear layer's bias
// gradient when A = dY) are written to csum[m], in a fixed order (per thread
// over the k-slices, then over 16 thread groups).
template <int AT, int BT, int EPI, bool CSUM = false>
__device__ __forceinline__ void big8_tile(const OpArgs& A, const OpArgs& B, int K, int kchunk,
                                          const EpiArgs& e, float* partial, int tx, int ty, int tz,
                                          bf16_t* smem, float* csum = nullptr) {
  static_assert(!CSUM || AT == 1, "column sums of a K-major A tile");
  // Stage s of A at s * 32 KB, of B at 64 KB + s * 32 KB: each operand's two
  // stages lie within one LDS instruction offset (16 bits) of each other.
  bf16_t* const sA0 = smem;
  bf16_t* const sA1 = smem + BIG * BK;
  bf16_t* const sB0 = smem + 2 * BIG * BK;
  bf16_t* const sB1 = smem + 3 * BIG * BK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;  // rows wm * 128 .., columns wn * 64 ..
  const int m0 = ty * BIG, n0 = tx * BIG;
  const int kbeg = tz * kchunk;
  if (EPI == EPI_PARTIAL) partial += (long)tz * e.M * e.N;
  const int kend = min(K, kbeg + kchunk);
  const int nk = (kend - kbeg + BK - 1) / BK;

  OpArgs a = A, b = B;
  a.kvalid = min(a.kvalid, kend);
  b.kvalid = min(b.kvalid, kend);
  const long a_extent = AT ? (long)a.kvalid * a.ld : (long)a.rows * a.ld;
  const long b_extent = BT ? (long)b.kvalid * b.ld : (long)b.rows * b.ld;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.X, a_extent * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(b.X, b_extent * 2);

  float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const bool do_cs = CSUM && csum != nullptr;
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // Full k-tiles load through the precomputed offsets; a ragged last one (and
  // the first, if ragged) through the masked loader.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  unsigned voa[4], vob[4];
  dma_plan256_w8<AT>(a, m0, kbeg, wave, lane, voa);
  dma_plan256_w8<BT>(b, n0, kbeg, wave, lane, vob);
  const unsigned a_kstep = AT ? (unsigned)(a.ld * 2 * BK) : 2u * BK;  // bytes per k-tile
  const unsigned b_kstep = BT ? (unsigned)(b.ld * 2 * BK) : 2u * BK;
  auto load_stage = [&](int kt, bf16_t* sa, bf16_t* sb) {
    const int k0 = kbeg + kt * BK;
    if (k0 + BK <= a.kvalid) dma_fast256_w8(ra, voa, (unsigned)kt * a_kstep, sa, wave_s);
    else dma_tile256_w8<AT, true>(ra, a, m0, k0, sa, wave, lane);
    if (k0 + BK <= b.kvalid) dma_fast256_w8(rb, vob, (unsigned)kt * b_kstep, sb, wave_s);
    else dma_tile256_w8<BT, true>(rb, b, n0, k0, sb, wave, lane);
  };
  load_stage(0, sA0, sB0);
  // One k-tile from stage ODD; the loop runs them in pairs so each stage's LDS
  // addresses are fixed offsets of loop-invariant registers.
  auto ktile = [&](int kt, auto odd_c) {
    constexpr bool odd = decltype(odd_c)::value;
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's loads of tile kt landed
    __syncthreads();                     // ... and every other wave's
    if (kt + 1 < nk) load_stage(kt + 1, odd ? sA0 : sA1, odd ? sB0 : sB1);
    const bf16_t* as = odd ? sA1 : sA0;
    const bf16_t* bs = odd ? sB1 : sB0;
    // Fragments double-buffered across the 16-deep steps: the reads of step
    // ks + 1 are issued between the MFMAs of step ks (the scheduling groups
    // pin that interleave), so no MFMA waits on an LDS read it could have had
    // one step earlier.
    constexpr int NDS = (AT ? 8 : 4) + (BT ? 4 : 2);  // LDS read instructions per step
    bf16x8 af[2][4], bf[2][2];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) af[0][i] = big_frag<AT>(as, wm * 128 + i * 32, 0, lane);
#pragma unroll
    for (int j = 0; j < 2; ++j) bf[0][j] = big_frag<BT>(bs, wn * 64 + j * 32, 0, lane);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[cur ^ 1][i] = big_frag<AT>(as, wm * 128 + i * 32, ks + 1, lane);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bf[cur ^ 1][j] = big_frag<BT>(bs, wn * 64 + j * 32, ks + 1, lane);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[cur][j], af[cur][i], acc[i][j], 0, 0, 0);
    }
    // schedule: step 0's reads, then per step its 8 MFMAs with the next
    // step's reads spread between them
    __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) sched_mfma_ds<8, NDS>();
      else __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (CSUM) {
      if (do_cs) {  // thread: 8 rows (chunk c), k-rows kg + 16 j of this slice
        const int c = threadIdx.x & 31, kg = threadIdx.x >> 5;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = kg + 16 * j;
          const u32x4 v = *(const u32x4*)(as + k * BIG + ((c ^ ((k & 3) << 2)) << 3));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            cs[2 * q] += bf_lo(v[q]);
            cs[2 * q + 1] += bf_hi(v[q]);
          }
        }
      }
    }
  };
  for (int kt = 0; kt < nk; kt += 2) {
    ktile(kt, std::false_type{});
    if (kt + 1 < nk) ktile(kt + 1, std::true_type{});
  }

  // Epilogue, one 32-row block of the wave's 128 x 64 tile at a time:
  // accumulators -> this wave's LDS slice as floats [32][CP], then each lane
  // applies the epilogue to 8 consecutive columns.  acc[i][j] = D[n][m]: lane
  // column m = lane % 32, register r holds n = 8 (r / 4) + 4 (lane / 32) + r % 4.
  constexpr int CP = 68;  // padded row pitch (floats)
  __syncthreads();        // every wave is done reading the operand tiles
  if constexpr (CSUM) {
    if (do_cs) {  // combine the 16 k-groups per row in LDS past the epilogue slices
      float* red = (float*)smem + 24576;
      const int c = threadIdx.x & 31, kg = threadIdx.x >> 5;
      *(float4*)(red + kg * 256 + 8 * c) = make_float4(cs[0], cs[1], cs[2], cs[3]);
      *(float4*)(red + kg * 256 + 8 * c + 4) = make_float4(cs[4], cs[5], cs[6], cs[7]);
      __syncthreads();
      if (threadIdx.x < 256) {
        float t = 0.f;
#pragma unroll
        for (int g = 0; g < 16; ++g) t += red[g * 256 + threadIdx.x];
        if (m0 + (int)threadIdx.x < e.M) csum[m0 + threadIdx.x] = t;
      }
    }
  }
  float* Cw = (float*)smem + wave * (32 * CP);  // 8 slices of 8.5 KB (68 KB of the 128 KB)
  const int m_l = lane & 31, nq = 4 * (lane >> 5);
  // The bias of this lane's 8 columns, loaded once for the tile (the
  // epilogue would reload it for every row block) and added here.
  constexpr bool BIAS_EPI = EPI == GPT_EPI_STORE || EPI == GPT_EPI_RESIDUAL ||
                            EPI == GPT_EPI_GELU || EPI == GPT_EPI_GELU_PAIR;
  float4 bias0 = make_float4(0.f, 0.f, 0.f, 0.f), bias1 = bias0;
  EpiArgs eb = e;
  bool has_bias = false;
  if constexpr (BIAS_EPI) {
    const int n = n0 + wn * 64 + (lane & 7) * 8;
    has_bias = e.bias != nullptr;
    if (has_bias && n < e.N) {
      bias0 = *(const float4*)(e.bias + n);
      bias1 = *(const float4*)(e.bias + n + 4);
    }
    eb.bias = nullptr;
  }
  // MUL: the 16 auxiliary vectors this lane multiplies by are loaded before
  // the blocks, so one memory round trip covers all of them.
  u32x4 pre[4][4];
  if constexpr (EPI == GPT_EPI_MUL) {
    const int n = n0 + wn * 64 + (lane & 7) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int m = m0 + wm * 128 + i * 32 + p * 8 + (lane >> 3);
        if (m < e.M && n < e.N)
          pre[i][p] = *(const u32x4*)((const bf16_t*)e.aux + (long)m * e.ldaux + n);
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(float4*)(Cw + m_l * CP + j * 32 + 8 * q + nq) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                        acc[i][j][4 * q + 3]);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
    const int cg = lane & 7;
    const int n = n0 + wn * 64 + cg * 8;
    // Unrolled: the four passes' auxiliary reads (GELU', residual) are
    // independent, so they are in flight together rather than one at a time.
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = p * 8 + (lane >> 3);
      const int m = m0 + wm * 128 + i * 32 + row;
      if (m < e.M && n < e.N) {
        float4 v0 = *(const float4*)(Cw + row * CP + cg * 8);
        float4 v1 = *(const float4*)(Cw + row * CP + cg * 8 + 4);
        if constexpr (EPI == GPT_EPI_MUL) {
          mul8_store(e, m, n, v0, v1, pre[i][p]);
        } else if constexpr (BIAS_EPI) {
          if (has_bias) {
            v0 = make_float4(v0.x + bias0.x, v0.y + bias0.y, v0.z + bias0.z, v0.w + bias0.w);
            v1 = make_float4(v1.x + bias1.x, v1.y + bias1.y, v1.z + bias1.z, v1.w + bias1.w);
          }
          epilogue8<EPI>(eb, partial, m, n, v0, v1);
        } else {
          epilogue8<EPI>(e, partial, m, n, v0, v1);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next block overwrites
  }
}

template <int AT, int BT, int EPI>
__global__ void __launch_bounds__(512, 1) gemm_big8_kernel(OpArgs A, OpArgs B, int K, int kchunk,
                                                           EpiArgs e, float* partial) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[4 * BIG * BK];
  int tx, ty, tz;
  xcd_tile(tx, ty, tz);
  if (e.batch > 1) {  // tz indexes the matrix of a batch (never split over K)
    batch_select(tz, A, B, e);
    tz = 0;
  }
  big8_tile<AT, BT, EPI>(A, B, K, kchunk, e, partial, tx, ty, tz, smem);
}

// ----------------------------------------------------------------------------
// bf16 MFMA, 256 x 192 tile, 8 waves of 64 x 96 (2 x 3 MFMA blocks): for
// N = 768 products (the residual-width outputs: M = tokens), whose 256 x 256
// grid is 192 tiles (three quarters of the CUs) and whose 128-tile grid is 1.5
// rounds, this grid is 256 tiles: one full round.  Stages, loaders and LDS
// layouts are the 256-tile kernel's (B rows past the tile are masked, so they
// are not fetched); the epilogue stages each wave's two 32 x 96 slices.
// ----------------------------------------------------------------------------
constexpr int BW = 192;

template <int AT, int BT, int EPI>
__global__ void __launch_bounds__(512, 1) gemm_big8w_kernel(OpArgs A, OpArgs B, int K, int kchunk,
                                                            EpiArgs e, float* partial) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[4 * BIG * BK];
  bf16_t* const sA0 = smem;  // stage layout of the 256-tile kernel
  bf16_t* const sA1 = smem + BIG * BK;
  bf16_t* const sB0 = smem + 2 * BIG * BK;
  bf16_t* const sB1 = smem + 3 * BIG * BK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // rows wm * 64 .., columns wn * 96 ..
  int tx, ty, tz;
  xcd_tile(tx, ty, tz);
  if (e.batch > 1) {  // tz indexes the matrix of a batch (never split over K)
    batch_select(tz, A, B, e);
    tz = 0;
  }
  const int m0 = ty * BIG, n0 = tx * BW;
  const int kbeg = tz * kchunk;
  if (EPI == EPI_PARTIAL) partial += (long)tz * e.M * e.N;
  const int kend = min(K, kbeg + kchunk);
  const int nk = (kend - kbeg + BK - 1) / BK;

  OpArgs a = A, b = B;
  a.kvalid = min(a.kvalid, kend);
  b.kvalid = min(b.kvalid, kend);
  const long a_extent = AT ? (long)a.kvalid * a.ld : (long)a.rows * a.ld;
  const long b_extent = BT ? (long)b.kvalid * b.ld : (long)b.rows * b.ld;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.X, a_extent * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(b.X, b_extent * 2);
  b.rows = min(b.rows, n0 + BW);  // the 256-row loader skips rows past this tile

  f32x16 acc[2][3];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[i][j] = f32x16{};

  // Full k-tiles through precomputed offsets, as in the 256-tile kernel.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  unsigned voa[4], vob[4];
  dma_plan256_w8<AT>(a, m0, kbeg, wave, lane, voa);
  dma_plan256_w8<BT>(b, n0, kbeg, wave, lane, vob);
  const unsigned a_kstep = AT ? (unsigned)(a.ld * 2 * BK) : 2u * BK;
  const unsigned b_kstep = BT ? (unsigned)(b.ld * 2 * BK) : 2u * BK;
  auto load_stage = [&](int kt, bf16_t* sa, bf16_t* sb) {
    const int k0 = kbeg + kt * BK;
    if (k0 + BK <= a.kvalid) dma_fast256_w8(ra, voa, (unsigned)kt * a_kstep, sa, wave_s);
    else dma_tile256_w8<AT, true>(ra, a, m0, k0, sa, wave, lane);
    if (k0 + BK <= b.kvalid) dma_fast256_w8(rb, vob, (unsigned)kt * b_kstep, sb, wave_s);
    else dma_tile256_w8<BT, true>(rb, b, n0, k0, sb, wave, lane);
  };
  load_stage(0, sA0, sB0);
  auto ktile = [&](int kt, auto odd_c) {  // k-tiles in pairs, as in the 256-tile kernel
    constexpr bool odd = decltype(odd_c)::value;
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's loads of tile kt landed
    __syncthreads();                     // ... and every other wave's
    if (kt + 1 < nk) load_stage(kt + 1, odd ? sA0 : sA1, odd ? sB0 : sB1);
    const bf16_t* as = odd ? sA1 : sA0;
    const bf16_t* bs = odd ? sB1 : sB0;
    // Fragments double-buffered across the 16-deep steps, as in the 256-tile kernel.
    constexpr int NDS = (AT ? 4 : 2) + (BT ? 6 : 3);
    bf16x8 af[2][2], bf[2][3];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2; ++i) af[0][i] = big_frag<AT>(as, wm * 64 + i * 32, 0, lane);
#pragma unroll
    for (int j = 0; j < 3; ++j) bf[0][j] = big_frag<BT>(bs, wn * 96 + j * 32, 0, lane);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[cur ^ 1][i] = big_frag<AT>(as, wm * 64 + i * 32, ks + 1, lane);
#pragma unroll
        for (int j = 0; j < 3; ++j)
          bf[cur ^ 1][j] = big_frag<BT>(bs, wn * 96 + j * 32, ks + 1, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[cur][j], af[cur][i], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) sched_mfma_ds<6, NDS>();
      else __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = 0; kt < nk; kt += 2) {
    ktile(kt, std::false_type{});
    if (kt + 1 < nk) ktile(kt + 1, std::true_type{});
  }

  // Epilogue, one 32-row block of the wave's 64 x 96 tile at a time (see the
  // 256-tile kernel): acc[i][j] = D[n][m], lane column m = lane % 32, register
  // r holds n = 8 (r / 4) + 4 (lane / 32) + r % 4; 12 groups of 8 columns per row.
  constexpr int CP = 100;  // padded row pitch (floats)
  __syncthreads();         // every wave is done reading the operand tiles
  float* Cw = (float*)smem + wave * (32 * CP);  // 8 slices of 12.5 KB (100 KB of the 128 KB)
  const int m_l = lane & 31, nq = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(float4*)(Cw + m_l * CP + j * 32 + 8 * q + nq) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                        acc[i][j][4 * q + 3]);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
#pragma unroll
    for (int p = 0; p < 6; ++p) {  // 32 rows x 12 column groups = 6 passes of 64 lanes
      const int item = p * 64 + lane, row = item / 12, cg = item - row * 12;
      const int m = m0 + wm * 64 + i * 32 + row, n = n0 + wn * 96 + cg * 8;
      if (m < e.M && n < e.N) {
        const float4 v0 = *(const float4*)(Cw + row * CP + cg * 8);
        const float4 v1 = *(const float4*)(Cw + row * CP + cg * 8 + 4);
        epilogue8<EPI>(e, partial, m, n, v0, v1);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next block overwrites
  }
}

MfmaKernel big8w_kernel_for(int at, int bt, int epi, int ga, int gb) {
  if (ga || gb) return nullptr;
#define K_(AT, BT, EP) \
  if (at == AT && bt == BT && epi == EP) return gemm_big8w_kernel<AT, BT, EP>;
  K_(0, 0, GPT_EPI_STORE)
  K_(0, 0, GPT_EPI_RESIDUAL)
  K_(0, 1, GPT_EPI_STORE)
  K_(0, 1, GPT_EPI_MUL)
  K_(0, 1, GPT_EPI_DGELU)
#undef K_
  return nullptr;
}

// Up to GROUP_MAX products with the same K (a transformer block's weight
// gradients: K = tokens) in one launch over their concatenated 256-tiles, each
// split S ways over K.  Workgroups walk the flat (split, tile) space in the
// XCD-contiguous order of `xcd_tile`; within a product, tiles go in groups of
// TILE_GROUP tile rows, column by column.
constexpr int GROUP_MAX = 4;
struct GroupArgs {
  OpArgs A[GROUP_MAX], B[GROUP_MAX];
  int M[GROUP_MAX], N[GROUP_MAX], nx[GROUP_MAX], ny[GROUP_MAX];
  int tile0[GROUP_MAX + 1];  // first flat tile of each product; tile0[n] = all tiles
  long part[GROUP_MAX];      // float offset of each product's S partial tiles
  float* csum[GROUP_MAX];    // NULL, or [S][M] partial column sums of A (bias gradient)
  int n;
};

template <int AT, int BT>
__global__ void __launch_bounds__(512, 1) gemm_big8_group_kernel(GroupArgs g, int K, int kchunk,
                                                                 float* partial) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[4 * BIG * BK];
  const int T = g.tile0[g.n];
  const int total = gridDim.x, L = blockIdx.x;
  const int id = (total & 7) == 0 ? (L & 7) * (total >> 3) + (L >> 3) : L;
  const int tz = id / T, t = id - tz * T;
  int p = 0;
  while (p + 1 < g.n && t >= g.tile0[p + 1]) ++p;
  const int r = t - g.tile0[p], nx = g.nx[p], ny = g.ny[p];
  const int grp = r / (TILE_GROUP * nx);
  const int rows = min(TILE_GROUP, ny - grp * TILE_GROUP);
  const int w = r - grp * TILE_GROUP * nx;
  EpiArgs e{};
  e.epi = EPI_PARTIAL;
  e.M = g.M[p];
  e.N = g.N[p];
  e.batch = 1;
  const int tx = w / rows;
  float* cs = (AT == 1 && tx == 0 && g.csum[p]) ? g.csum[p] + (long)tz * e.M : nullptr;
  big8_tile<AT, BT, EPI_PARTIAL, AT == 1>(g.A[p], g.B[p], K, kchunk, e, partial + g.part[p], tx,
                                          grp * TILE_GROUP + w % rows, tz, smem, cs);
}

MfmaKernel big8_kernel_for(int at, int bt, int epi, int ga, int gb) {
  if (ga || gb) return nullptr;
#define K_(AT, BT, EP) \
  if (at == AT && bt == BT && epi == EP) return gemm_big8_kernel<AT, BT, EP>;
  K_(0, 0, GPT_EPI_STORE)
  K_(0, 0, GPT_EPI_RESIDUAL)
  K_(0, 0, GPT_EPI_GELU)
  K_(0, 0, GPT_EPI_GELU_PAIR)
  K_(0, 0, GPT_EPI_F32)
  K_(0, 0, GPT_EPI_F32_ACCUM)
  K_(0, 0, GPT_EPI_DGELU)
  K_(0, 1, GPT_EPI_STORE)
  K_(0, 1, GPT_EPI_DGELU)
  K_(0, 1, GPT_EPI_MUL)
  K_(0, 1, GPT_EPI_F32)
  K_(0, 1, EPI_PARTIAL)
  K_(0, 0, GPT_EPI_AXPBY)
  K_(0, 1, GPT_EPI_AXPBY)
  K_(1, 1, GPT_EPI_STORE)
  K_(1, 1, GPT_EPI_F32)
  K_(1, 1, GPT_EPI_F32_ACCUM)
  K_(1, 1, EPI_PARTIAL)
#undef K_
  return nullptr;
}

int choose_split(int M, int N, int K) {
  long tiles = cdiv(M, BM) * cdiv(N, BN);
  if (tiles >= 512 || K < 1024) return 1;
  int s = (int)cdiv(1024, tiles);
  int maxs = K / 512;
  if (s > maxs) s = maxs;
  if (s > 32) s = 32;
  return s < 1 ? 1 : s;
}

// Which kernel runs a descriptor and over how many K splits.
struct GemmPlan {
  bool big;   // 256 x 256 tiles
  int S;      // K splits (1 = none)
  bool wide;  // 256 x 192 tiles (unsplit)
};

GemmPlan plan_gemm(int M, int N, int K, int precision, bool splittable, int64_t ws_bytes,
                   bool big_ok, int batch = 1, bool wide_ok = false, int side_by_side = 1) {
  GemmPlan p{false, 1, false};
  if (precision != GPT_BF16 || M <= 0 || N <= 0 || K <= 0) return p;
  if (!big_ok) {
    int S = splittable ? choose_split(M, N, K) : 1;
    if (S > 1 && ws_bytes < (int64_t)S * M * N * 4) S = 1;
    p.S = S;
    return p;
  }
  // Few rows (decode steps: one row per sequence): one row of 128-tiles, so the
  // weight matrix is streamed by as many workgroups as K splits allow.
  if (splittable && batch == 1 && M <= BM) {
    const long t128 = cdiv(N, BN);
    if (t128 < 256) {
      int S = (int)std::min<long>(std::min<long>(32, K / BK), cdiv(512, t128));
      if (S > 1 && ws_bytes >= (int64_t)S * M * N * 4) {
        p.S = S;
        return p;
      }
    }
  }
  // Grids of unsplit products that run side by side (batch chains of the
  // forward) fill the CUs together: their fill is judged on all their tiles.
  const long cf = splittable ? 1 : std::max(1, side_by_side);
  const long t256 = cdiv(M, BIG) * cdiv(N, BIG) * batch * cf;
  // 256 x 192 tiles where that grid fills whole rounds of the 256 CUs and the
  // square grids do not (N = 768: 256 tiles against 192 of 256 x 256 and 1.5
  // rounds of 128 x 128; QKV forward: 3 rounds).  Not for products that may be
  // split over K (the vocabulary input gradient is 4% faster split 4 ways on
  // 256-tiles than unsplit here).
  if (wide_ok && !splittable && batch == 1) {
    auto fill = [](long t, long slots) { return (double)t / (double)(cdiv(t, slots) * slots); };
    const long t192 = cdiv(M, BIG) * cdiv(N, BW) * cf, t128 = cdiv(M, BM) * cdiv(N, BN) * cf;
    const double f192 = fill(t192, 256);
    if (t192 >= 256 && f192 >= 0.95 && f192 > std::max(fill(t256, 256), fill(t128, 512)) + 0.05) {
      p.wide = true;
      return p;
    }
  }
  {
    // Long reductions over few output tiles (weight gradients: K = tokens; the
    // vocabulary projection's input gradient: K = vocabulary): 256-tiles with
    // K split, the split count the one that needs the fewest rounds of the 256
    // CUs per unit of work (the smallest such).
    if (splittable && K >= 2048 && t256 < 256) {
      const int maxs = (int)std::min<long>(K / 1024, 32);
      int S = 1;
      double best = 1.0;  // rounds per split of the unsplit grid: cdiv(t256, 256) / 1
      for (int c = 2; c <= maxs; ++c) {
        const double r = (double)cdiv(t256 * c, 256) / c;
        if (r < best - 1e-9) {
          best = r;
          S = c;
        }
      }
      if (S >= 2 && ws_bytes >= (int64_t)S * M * N * 4) {
        p.big = true;
        p.S = S;
        return p;
      }
    }
    // Long reductions over many output tiles (the vocabulary weight gradient:
    // K = tokens, 591 tiles): unsplit 256-tiles.  Alone this is 3% slower than
    // 128-tiles (the last of three rounds is a third full), but it runs beside
    // the input-gradient chain, which fills those CUs: +1.1% on the step.
    if (splittable && K >= 2048 && t256 >= 256) {
      p.big = true;
      return p;
    }
    // The vocabulary projection and its input gradient (N or K = vocabulary): 256-tiles.
    if (!splittable && (t256 >= 4096 || K >= 16384)) {
      p.big = true;
      return p;
    }
    // Otherwise 256-tiles (one workgroup per CU) when they fill the rounds of
    // the 256 CUs at least as evenly as 128-tiles (two workgroups per CU) do;
    // on a tie below full rounds with a short reduction (K <= 1024) the
    // 128-tiles, whose two workgroups per CU hide each other's epilogue
    // (measured on the 768 x 768 projections; at full rounds, e.g. the
    // 3072-wide FC products, the 256-tiles stay faster).
    if (!splittable && t256 >= 128) {
      const long t128 = cdiv(M, BM) * cdiv(N, BN) * batch * cf;
      const double f256 = (double)t256 / (256.0 * cdiv(t256, 256));
      const double f128 = (double)t128 / (512.0 * cdiv(t128, 512));
      const bool tie = f256 < f128 + 1e-9 && f256 < 1.0 - 1e-9;
      if (f256 + 1e-9 >= f128 && !(tie && K <= 1024)) {
        p.big = true;
        return p;
      }
    }
  }
  int S = splittable ? choose_split(M, N, K) : 1;
  if (S > 1 && ws_bytes < (int64_t)S * M * N * 4) S = 1;
  p.S = S;
  return p;
}

int effective_splits(const GemmPlan& p, int K) {
  if (p.S <= 1) return 1;
  const int kchunk = (int)cdiv(cdiv(K, p.S), BK) * BK;
  return (int)cdiv(K, kchunk);
}

// K may be split (partials reduced, epilogue applied after) for weight
// gradients, for very long reductions and for products of at most 128 rows.
bool splittable(const gpt_gemm_desc& d) {
  return !d.a_gelu && !d.b_gelu && ((d.a_trans && d.b_trans) || d.K >= 16384 || d.M <= BM);
}
// Direct-to-LDS loads address each operand through a 31-bit byte offset.
bool dma_ok(const gpt_gemm_desc& d) {
  const long ea = d.a_trans ? (long)d.a_kvalid * d.lda : (long)d.a_rows * d.lda;
  const long eb = d.b_trans ? (long)d.b_kvalid * d.ldb : (long)d.b_rows * d.ldb;
  return ea * 2 < 0x7fffffffL && eb * 2 < 0x7fffffffL;
}
// The large-tile kernel loads straight to LDS, so it cannot apply GELU to an
// operand on the way in.
bool big_ok(const gpt_gemm_desc& d) { return !d.a_gelu && !d.b_gelu && dma_ok(d); }
// The 256 x 192 kernel has the layout / epilogue combination and vector stores apply.
bool wide_ok(const gpt_gemm_desc& d) {
  const bool vec = d.N % 8 == 0 && d.ldo % 8 == 0 && (d.aux == nullptr || d.ldaux % 8 == 0);
  return vec && d.batch <= 1 && big_ok(d) &&
         big8w_kernel_for(d.a_trans, d.b_trans, d.epilogue, d.a_gelu, d.b_gelu) != nullptr;
}

}  // namespace

int gemm_split_count(const gpt_gemm_desc& d, int side_by_side) {
  GemmPlan p = plan_gemm(d.M, d.N, d.K, d.precision, splittable(d),
                         d.workspace ? d.workspace_bytes : 0, big_ok(d), 1, wide_ok(d),
                         side_by_side);
  return effective_splits(p, d.K);
}

int64_t gemm_workspace_bytes(int M, int N, int K, int precision) {
  GemmPlan p = plan_gemm(M, N, K, precision, true, INT64_MAX, true);
  GemmPlan q = plan_gemm(M, N, K, precision, true, INT64_MAX, false);
  const int S = std::max(p.S, q.S);
  return S > 1 ? (int64_t)S * M * N * 4 : 0;
}

hipError_t gemm(const gpt_gemm_desc& d, hipStream_t s, int side_by_side) {
  if (d.M <= 0 || d.N <= 0) return hipSuccess;
  // Vector loads: 8 K-values (row-major operand) or 8 rows (K-major operand).
  const bool k_vectors = !d.a_trans || !d.b_trans;
  if (d.K < 0 || (k_vectors && d.K % 8) || (d.lda % 8) || (d.ldb % 8)) return hipErrorInvalidValue;
  const int batch = d.batch > 1 ? d.batch : 1;
  if (batch > 1 && (d.bias || d.resid)) return hipErrorInvalidValue;
  EpiArgs e{d.epilogue, d.gelu_tanh, d.M,      d.N,        d.bias,       d.resid,
            d.out,      d.ldo,       d.aux,    d.ldaux,    d.alpha,      d.beta,
            batch,      d.stride_a,  d.stride_b, d.stride_out, d.stride_aux};
  OpArgs A{d.A, d.lda, d.a_trans, d.a_rows, d.a_kvalid, d.a_gelu};
  OpArgs B{d.B, d.ldb, d.b_trans, d.b_rows, d.b_kvalid, d.b_gelu};
  if (d.K == 0) {
    // Empty reduction: the epilogue still runs on a zero accumulator.
    dim3 grid((unsigned)cdiv(d.N, 64), (unsigned)cdiv(d.M, 64), (unsigned)batch);
    if (d.precision == GPT_BF16)
      gemm_simt_kernel<bf16_t, bf16_t><<<grid, 256, 0, s>>>(A, B, 0, e);
    else
      gemm_simt_kernel<float, float><<<grid, 256, 0, s>>>(A, B, 0, e);
    return hipGetLastError();
  }
  if (d.precision != GPT_BF16) {
    dim3 grid((unsigned)cdiv(d.N, 64), (unsigned)cdiv(d.M, 64), (unsigned)batch);
    gemm_simt_kernel<float, float><<<grid, 256, 0, s>>>(A, B, d.K, e);
    return hipGetLastError();
  }
  const GemmPlan plan = plan_gemm(d.M, d.N, d.K, d.precision, batch == 1 && splittable(d),
                                  d.workspace ? d.workspace_bytes : 0, big_ok(d), batch,
                                  wide_ok(d), side_by_side);
  if (plan.wide) {  // wide_ok: the kernel exists for this combination
    dim3 grid((unsigned)cdiv(d.N, BW), (unsigned)cdiv(d.M, BIG), 1);
    big8w_kernel_for(d.a_trans, d.b_trans, d.epilogue, 0, 0)<<<grid, 512, 0, s>>>(A, B, d.K, d.K,
                                                                                  e, nullptr);
    return hipGetLastError();
  }
  const int S = effective_splits(plan, d.K);
  const bool vec_ok = d.N % 8 == 0 && d.ldo % 8 == 0 && (d.aux == nullptr || d.ldaux % 8 == 0);
  const int epi = S > 1 ? EPI_PARTIAL : d.epilogue;
  // 256-tiles run the 8-wave kernel; a combination it lacks drops to the
  // 128-tile kernels (the split plan and its partials do not depend on the tile).
  MfmaKernel kern = nullptr;
  int threads = 256;
  bool big = plan.big;
  if (vec_ok) {
    if (big) {
      kern = big8_kernel_for(d.a_trans, d.b_trans, epi, d.a_gelu, d.b_gelu);
      threads = 512;
      if (kern == nullptr) {
        big = false;
        threads = 256;
      }
    }
    if (!big) {
      kern = mfma_kernel_for(d.a_trans, d.b_trans, epi, d.a_gelu, d.b_gelu);
      if (dma_ok(d)) {
        MfmaKernel k2 = dma_kernel_for(d.a_trans, d.b_trans, epi, d.a_gelu, d.b_gelu);
        if (k2) kern = k2;
      }
    }
  }
  if (kern == nullptr) {
    // Combinations the step never issues: the generic kernel (bf16 inputs).
    dim3 grid((unsigned)cdiv(d.N, 64), (unsigned)cdiv(d.M, 64), (unsigned)batch);
    gemm_simt_kernel<bf16_t, bf16_t><<<grid, 256, 0, s>>>(A, B, d.K, e);
    return hipGetLastError();
  }
  const int T = big ? BIG : BM;
  dim3 grid((unsigned)cdiv(d.N, T), (unsigned)cdiv(d.M, T), (unsigned)(S * batch));
  if (S == 1) {
    kern<<<grid, threads, 0, s>>>(A, B, d.K, d.K, e, nullptr);
    return hipGetLastError();
  }
  const int kchunk = (int)cdiv(cdiv(d.K, plan.S), BK) * BK;
  kern<<<grid, threads, 0, s>>>(A, B, d.K, kchunk, e, (float*)d.workspace);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  long total = (long)d.M * d.N;
  const float* ws = (const float*)d.workspace;
  if (vec_ok && (d.epilogue == GPT_EPI_F32 || d.epilogue == GPT_EPI_F32_ACCUM ||
                 d.epilogue == GPT_EPI_STORE)) {
    const unsigned blocks = (unsigned)std::min<long>(cdiv(total / 8, 256), 4096);
    if (d.epilogue == GPT_EPI_F32)
      splitk_reduce8_kernel<GPT_EPI_F32><<<blocks, 256, 0, s>>>(ws, S, e);
    else if (d.epilogue == GPT_EPI_F32_ACCUM)
      splitk_reduce8_kernel<GPT_EPI_F32_ACCUM><<<blocks, 256, 0, s>>>(ws, S, e);
    else
      splitk_reduce8_kernel<GPT_EPI_STORE><<<blocks, 256, 0, s>>>(ws, S, e);
    return hipGetLastError();
  }
  unsigned blocks = (unsigned)std::min<long>(cdiv(total, 256), 4096);
  splitk_reduce_kernel<bf16_t><<<blocks, 256, 0, s>>>(ws, S, e);
  return hipGetLastError();
}

namespace {
// out[m] (+)= sum_k A(m, k) of a K-major bf16 operand, k in order (the
// bias gradients of products the grouped kernel does not take).
__global__ void __launch_bounds__(256) csum_kmajor_kernel(const bf16_t* __restrict__ A, long lda,
                                                          int M, int K, float* __restrict__ out,
                                                          int accumulate) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  float t = 0.f;
  for (int k = 0; k < K; ++k) t += bf2f(A[(long)k * lda + m]);
  out[m] = accumulate ? out[m] + t : t;
}

// Every reduction of a grouped launch in one kernel: work item i < vec_end
// sums 8 consecutive outputs of product p over the S splits (split order) and
// stores or adds them; items past vec_end do the same for one bias-gradient
// element.  Same sums, in the same order, as one reduction per product.
struct GroupReduceArgs {
  const float* part[GROUP_MAX];
  float* out[GROUP_MAX];
  long ldo[GROUP_MAX];
  int M[GROUP_MAX], N[GROUP_MAX];
  long vec0[GROUP_MAX + 1];  // first vector item of each product; vec0[n]: all
  const float* cpart[GROUP_MAX];  // the nc bias gradients: partials [S][M] and outputs
  float* db[GROUP_MAX];
  int cM[GROUP_MAX];
  long c0[GROUP_MAX + 1];  // first item of each bias gradient (c0[0] = vec0[n]); c0[nc]: all
  int n, nc, S, accumulate;
  double* sq;  // NULL, or one sum of squares of the written values per block
};

__global__ void __launch_bounds__(256) group_reduce_kernel(GroupReduceArgs r) {
  __shared__ double red[256];
  const long total = r.c0[r.nc];
  float ss = 0.f;  // this thread's sum of squares of what it writes (fixed order)
  for (long i = blockIdx.x * 256L + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    if (i < r.vec0[r.n]) {
      int p = 0;
      while (p + 1 < r.n && i >= r.vec0[p + 1]) ++p;
      const long j = i - r.vec0[p], per_row = r.N[p] / 8, plane = (long)r.M[p] * r.N[p];
      const int m = (int)(j / per_row), n = (int)(j % per_row) * 8;
      const float* q = r.part[p] + (long)m * r.N[p] + n;
      float4 a = *(const float4*)q, b = *(const float4*)(q + 4);
      for (int z = 1; z < r.S; ++z) {
        const float4 c = *(const float4*)(q + z * plane), d = *(const float4*)(q + z * plane + 4);
        a.x += c.x; a.y += c.y; a.z += c.z; a.w += c.w;
        b.x += d.x; b.y += d.y; b.z += d.z; b.w += d.w;
      }
      float4* o = (float4*)(r.out[p] + (long)m * r.ldo[p] + n);
      if (r.accumulate) {
        const float4 u = o[0], v = o[1];
        a = make_float4(u.x + a.x, u.y + a.y, u.z + a.z, u.w + a.w);
        b = make_float4(v.x + b.x, v.y + b.y, v.z + b.z, v.w + b.w);
      }
      o[0] = a;
      o[1] = b;
      ss += ((a.x * a.x + a.y * a.y) + (a.z * a.z + a.w * a.w)) +
            ((b.x * b.x + b.y * b.y) + (b.z * b.z + b.w * b.w));
    } else {
      int p = 0;
      while (p + 1 < r.nc && i >= r.c0[p + 1]) ++p;
      const int m = (int)(i - r.c0[p]);
      float t = r.cpart[p][m];
      for (int z = 1; z < r.S; ++z) t += r.cpart[p][(long)z * r.cM[p] + m];
      if (r.accumulate) t += r.db[p][m];
      r.db[p][m] = t;
      ss += t * t;
    }
  }
  if (r.sq) {  // block sum in double, in a fixed tree order
    red[threadIdx.x] = (double)ss;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) r.sq[blockIdx.x] = red[0];
  }
}
}  // namespace

namespace {
// Split count of a grouped launch over T 256-tiles: at most one (split, tile)
// workgroup per CU, each split at least 1024 deep.
int group_splits(long T, int K) {
  int S = (int)std::max<long>(1, 256 / std::max<long>(T, 1));
  return std::min(S, std::max(1, K / 1024));
}

long group_tiles(const int* M, const int* N, int n) {
  long T = 0;
  for (int i = 0; i < n; ++i) T += cdiv(M[i], BIG) * cdiv(N[i], BIG);
  return T;
}

// The grouped kernel's conditions: bf16, both operands K-major, fp32 output
// (store or accumulate, the same for all), one K, vector-width leading
// dimensions, operands within the 31-bit buffer offsets.
bool group_ok(const gpt_gemm_desc* d, int n) {
  if (n < 1 || n > GROUP_MAX) return false;
  for (int i = 0; i < n; ++i) {
    const gpt_gemm_desc& x = d[i];
    if (x.precision != GPT_BF16 || !x.a_trans || !x.b_trans || x.a_gelu || x.b_gelu) return false;
    if (x.batch > 1 || x.bias || x.resid || x.K != d[0].K || x.epilogue != d[0].epilogue) return false;
    if (x.epilogue != GPT_EPI_F32 && x.epilogue != GPT_EPI_F32_ACCUM) return false;
    if (x.M <= 0 || x.N <= 0 || x.K <= 0 || x.N % 8 || x.ldo % 8 || x.lda % 8 || x.ldb % 8) return false;
    if (!dma_ok(x)) return false;
  }
  return true;
}
}  // namespace

int64_t gemm_group_workspace_bytes(const int* M, const int* N, int n, int K) {
  if (n < 1 || n > GROUP_MAX) return 0;
  const int S = group_splits(group_tiles(M, N, n), K);
  int64_t mn = 0;
  for (int i = 0; i < n; ++i) mn += (int64_t)M[i] * N[i] + M[i];  // product + column-sum partials
  return (int64_t)S * mn * 4;
}

hipError_t gemm_group(const gpt_gemm_desc* d, int n, hipStream_t s, float* const* db, int phase,
                      double* sq) {
  if (n <= 0) return hipSuccess;
  const bool run_products = phase != 2, run_reduce = phase != 1;
  if (db) {  // column sums need a bf16 K-major A
    for (int i = 0; i < n; ++i)
      if (db[i] && (d[i].precision != GPT_BF16 || !d[i].a_trans || d[i].a_gelu))
        return hipErrorInvalidValue;
  }
  int Ms[GROUP_MAX], Ns[GROUP_MAX];
  bool grouped = group_ok(d, n);
  if (grouped) {
    for (int i = 0; i < n; ++i) {
      Ms[i] = d[i].M;
      Ns[i] = d[i].N;
    }
    grouped = d[0].workspace &&
              d[0].workspace_bytes >= gemm_group_workspace_bytes(Ms, Ns, n, d[0].K);
  }
  if (!grouped) {  // one launch per product, each with its own plan
    if (!run_products) return hipSuccess;
    for (int i = 0; i < n; ++i) {
      hipError_t e = gemm(d[i], s);
      if (e != hipSuccess) return e;
      if (db && db[i] && d[i].M > 0) {
        csum_kmajor_kernel<<<(unsigned)cdiv(d[i].M, 256), 256, 0, s>>>(
            (const bf16_t*)d[i].A, d[i].lda, d[i].M, d[i].K, db[i],
            d[i].epilogue == GPT_EPI_F32_ACCUM);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
    return hipSuccess;
  }
  const int K = d[0].K;
  const long T = group_tiles(Ms, Ns, n);
  const int S0 = group_splits(T, K);
  const int kchunk = (int)cdiv(cdiv(K, S0), BK) * BK;
  const int S = (int)cdiv(K, kchunk);
  GroupArgs g{};
  g.n = n;
  long tile = 0, part = 0;
  for (int i = 0; i < n; ++i) {
    const gpt_gemm_desc& x = d[i];
    g.A[i] = OpArgs{x.A, x.lda, 1, x.a_rows, x.a_kvalid, 0};
    g.B[i] = OpArgs{x.B, x.ldb, 1, x.b_rows, x.b_kvalid, 0};
    g.M[i] = x.M;
    g.N[i] = x.N;
    g.nx[i] = (int)cdiv(x.N, BIG);
    g.ny[i] = (int)cdiv(x.M, BIG);
    g.tile0[i] = (int)tile;
    g.part[i] = part;
    tile += (long)g.nx[i] * g.ny[i];
    part += (long)S * x.M * x.N;
  }
  g.tile0[n] = (int)tile;
  float* ws = (float*)d[0].workspace;
  for (int i = 0; i < n; ++i) {  // column-sum partials after the product partials
    g.csum[i] = (db && db[i]) ? ws + part : nullptr;
    part += (long)S * d[i].M;
  }
  if (run_products) {
    gemm_big8_group_kernel<1, 1><<<(unsigned)(T * S), 512, 0, s>>>(g, K, kchunk, ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || !run_reduce) return err;
  }
  // Each product's partials (and bias partials) summed in split order, one launch.
  GroupReduceArgs r{};
  r.n = n;
  r.S = S;
  r.accumulate = d[0].epilogue == GPT_EPI_F32_ACCUM;
  long items = 0;
  for (int i = 0; i < n; ++i) {
    r.part[i] = ws + g.part[i];
    r.out[i] = (float*)d[i].out;
    r.ldo[i] = d[i].ldo;
    r.M[i] = d[i].M;
    r.N[i] = d[i].N;
    r.vec0[i] = items;
    items += (long)d[i].M * d[i].N / 8;
  }
  r.vec0[n] = items;
  r.nc = 0;
  for (int i = 0; i < n; ++i) {  // the products with a bias gradient, in product order
    if (!g.csum[i]) continue;
    r.cpart[r.nc] = g.csum[i];
    r.db[r.nc] = db[i];
    r.cM[r.nc] = d[i].M;
    r.c0[r.nc] = items;
    items += d[i].M;
    ++r.nc;
  }
  r.c0[r.nc] = items;
  r.sq = sq;
  const unsigned blocks = (unsigned)std::min<long>(cdiv(items, 256), GROUP_REDUCE_MAX_BLOCKS);
  group_reduce_kernel<<<blocks, 256, 0, s>>>(r);
  return hipGetLastError();
}

int gemm_group_reduce_blocks(const gpt_gemm_desc* d, int n, float* const* db) {
  if (n <= 0 || !group_ok(d, n)) return 0;
  int Ms[GROUP_MAX], Ns[GROUP_MAX];
  long items = 0;
  for (int i = 0; i < n; ++i) {
    Ms[i] = d[i].M;
    Ns[i] = d[i].N;
    items += (long)d[i].M * d[i].N / 8 + ((db && db[i]) ? d[i].M : 0);
  }
  if (!d[0].workspace || d[0].workspace_bytes < gemm_group_workspace_bytes(Ms, Ns, n, d[0].K))
    return 0;
  return (int)std::min<long>(cdiv(items, 256), GROUP_REDUCE_MAX_BLOCKS);
}

}  // namespace gpt
