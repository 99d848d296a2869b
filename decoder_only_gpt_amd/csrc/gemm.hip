// Matrix products of the GPT step: C = op(A) . op(B)^T with fused epilogues.
//
// Every Linear layer of the model (nanoGPT README: "model.py ... a GPT model
// definition"; nanochat "FLOPs-Berechnung im Detail": each matmul parameter
// costs 2 FLOPs forward and 4 backward) runs through here three times:
//   forward  y  = x W^T            A = x  [M,K]            B = W [N,K]
//   backward dx = dy W             A = dy [M,K]            B = W stored [K,N]
//   backward dW = dy^T x           A = dy stored [K,M]     B = x stored [K,N]
//
// bf16 path: CDNA4 MFMA (v_mfma_f32_32x32x16_bf16), 128x128 output tile per
// 256-thread workgroup (2x2 waves of 64x64), K staged through LDS in 64-wide
// slices with double buffering.  Operands stored K-major are transposed in
// registers (4x8 blocks) on their way into LDS so every MFMA fragment is one
// 16-byte LDS read.  Long-K products (the weight gradients, K = B*T) are split
// over K into float partial tiles that a second kernel sums in a fixed order,
// so results are bitwise reproducible.
// fp32 path: a plain LDS-tiled FMA kernel (correctness path; small shapes).

#include "common.h"
#include "kernels.h"

#include <algorithm>

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
constexpr int LDS_PITCH = BK + 8;  // bf16 elements per LDS row (16-byte pad)

__device__ __forceinline__ u32x4 gelu_vec(u32x4 v, int tanh_form) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = pack_bf2(gelu_f(bf_lo(w[i]), tanh_form), gelu_f(bf_hi(w[i]), tanh_form));
  return u32x4{w[0], w[1], w[2], w[3]};
}

// Global -> registers for one BK-slice of a 128-row operand tile.
// Non-transposed: 4 vectors of 8 K-contiguous values per thread.
// Transposed (stored [k][r]): each thread loads 4 k-rows x 8 r-values.
struct Stage { u32x4 v[4]; };

__device__ __forceinline__ void stage_load(const OpArgs& a, int r0, int k0, int tanh_form,
                                           Stage& st) {
  const int t = threadIdx.x;
  const bf16_t* X = (const bf16_t*)a.X;
  if (!a.trans) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int vix = t + 256 * i;
      int row = vix >> 3, kv = vix & 7;
      int r = r0 + row, k = k0 + kv * 8;
      u32x4 val = {0, 0, 0, 0};
      if (r < a.rows && k < a.kvalid) val = *(const u32x4*)(X + (long)r * a.ld + k);
      st.v[i] = val;
    }
  } else {
    int blk = t >> 1, half = t & 1;
    int kb = blk >> 4, rb = blk & 15;
    int r = r0 + rb * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int k = k0 + kb * 8 + half * 4 + i;
      u32x4 val = {0, 0, 0, 0};
      if (r < a.rows && k < a.kvalid) val = *(const u32x4*)(X + (long)k * a.ld + r);
      st.v[i] = val;
    }
  }
  if (a.gelu) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st.v[i] = gelu_vec(st.v[i], tanh_form);
  }
}

__device__ __forceinline__ void stage_store(const OpArgs& a, const Stage& st, bf16_t* lds) {
  const int t = threadIdx.x;
  if (!a.trans) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int vix = t + 256 * i;
      int row = vix >> 3, kv = vix & 7;
      *(u32x4*)(lds + row * LDS_PITCH + kv * 8) = st.v[i];
    }
  } else {
    int blk = t >> 1, half = t & 1;
    int kb = blk >> 4, rb = blk & 15;
    // st.v[i] holds k = kb*8+half*4+i, r = rb*8 + 0..7.  Row r of the LDS tile
    // takes the 4 k-values {v[0][r], v[1][r], v[2][r], v[3][r]}.
    const uint32_t* w0 = (const uint32_t*)&st.v[0];
    const uint32_t* w1 = (const uint32_t*)&st.v[1];
    const uint32_t* w2 = (const uint32_t*)&st.v[2];
    const uint32_t* w3 = (const uint32_t*)&st.v[3];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // r pairs (2j, 2j+1)
      uint32_t lo01 = (w0[j] & 0xffffu) | (w1[j] << 16);
      uint32_t lo23 = (w2[j] & 0xffffu) | (w3[j] << 16);
      uint32_t hi01 = (w0[j] >> 16) | (w1[j] & 0xffff0000u);
      uint32_t hi23 = (w2[j] >> 16) | (w3[j] & 0xffff0000u);
      int row = rb * 8 + 2 * j;
      int col = kb * 8 + half * 4;
      *(uint2*)(lds + row * LDS_PITCH + col) = make_uint2(lo01, lo23);
      *(uint2*)(lds + (row + 1) * LDS_PITCH + col) = make_uint2(hi01, hi23);
    }
  }
}

template <bool SPLIT>
__global__ void __launch_bounds__(256, 2) gemm_mfma_kernel(OpArgs A, OpArgs B, int K, int kchunk,
                                                           EpiArgs e, float* partial) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDS_PITCH];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDS_PITCH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int kbeg = blockIdx.z * kchunk;
  const int kend = min(K, kbeg + kchunk);
  const int nk = (kend - kbeg + BK - 1) / BK;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // The K range of this split is [kbeg, kend); clamp operand validity to it.
  OpArgs a = A, b = B;
  a.kvalid = min(a.kvalid, kend);
  b.kvalid = min(b.kvalid, kend);

  Stage sa, sb;
  stage_load(a, m0, kbeg, e.tanh_form, sa);
  stage_load(b, n0, kbeg, e.tanh_form, sb);
  stage_store(a, sa, As[0]);
  stage_store(b, sb, Bs[0]);
  __syncthreads();

  const int frow = lane & 31, fk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      stage_load(a, m0, kbeg + (kt + 1) * BK, e.tanh_form, sa);
      stage_load(b, n0, kbeg + (kt + 1) * BK, e.tanh_form, sb);
    }
    const bf16_t* as = As[cur];
    const bf16_t* bs = Bs[cur];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *(const bf16x8*)(as + (wm * 64 + i * 32 + frow) * LDS_PITCH + ks * 16 + fk);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *(const bf16x8*)(bs + (wn * 64 + j * 32 + frow) * LDS_PITCH + ks * 16 + fk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      stage_store(a, sa, As[cur ^ 1]);
      stage_store(b, sb, Bs[cur ^ 1]);
    }
    __syncthreads();
  }

  // Accumulator layout of a 32x32 MFMA block: column = lane % 32,
  // row = 8 * (r / 4) + 4 * (lane / 32) + r % 4.
  const int g = lane >> 5, col = lane & 31;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        int n = n0 + wn * 64 + j * 32 + col;
        if (SPLIT) {
          if (m < e.M && n < e.N) partial[((long)blockIdx.z * e.M + m) * e.N + n] = acc[i][j][r];
        } else {
          epilogue<bf16_t>(e, m, n, acc[i][j][r]);
        }
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

int choose_split(int M, int N, int K) {
  long tiles = cdiv(M, BM) * cdiv(N, BN);
  if (tiles >= 512 || K < 1024) return 1;
  int s = (int)cdiv(1024, tiles);
  int maxs = K / 512;
  if (s > maxs) s = maxs;
  if (s > 32) s = 32;
  return s < 1 ? 1 : s;
}

}  // namespace

int gemm_split_count(const gpt_gemm_desc& d) {
  if (d.precision != GPT_BF16 || d.M <= 0 || d.N <= 0 || d.K <= 0) return 1;
  int S = choose_split(d.M, d.N, d.K);
  if (S > 1 && (d.workspace == nullptr || d.workspace_bytes < (int64_t)S * d.M * d.N * 4)) S = 1;
  if (S == 1) return 1;
  int kchunk = (int)cdiv(cdiv(d.K, S), BK) * BK;
  return (int)cdiv(d.K, kchunk);
}

int64_t gemm_workspace_bytes(int M, int N, int K, int precision) {
  if (precision != GPT_BF16) return 0;
  int s = choose_split(M, N, K);
  return s > 1 ? (int64_t)s * M * N * 4 : 0;
}

hipError_t gemm(const gpt_gemm_desc& d, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return hipSuccess;
  // Vector loads: 8 K-values (row-major operand) or 8 rows (K-major operand).
  const bool k_vectors = !d.a_trans || !d.b_trans;
  if (d.K < 0 || (k_vectors && d.K % 8) || (d.lda % 8) || (d.ldb % 8)) return hipErrorInvalidValue;
  EpiArgs e{d.epilogue, d.gelu_tanh, d.M, d.N, d.bias, d.resid, d.out, d.ldo, d.aux, d.ldaux};
  OpArgs A{d.A, d.lda, d.a_trans, d.a_rows, d.a_kvalid, d.a_gelu};
  OpArgs B{d.B, d.ldb, d.b_trans, d.b_rows, d.b_kvalid, d.b_gelu};
  if (d.K == 0) {
    // Empty reduction: the epilogue still runs on a zero accumulator.
    dim3 grid((unsigned)cdiv(d.N, 64), (unsigned)cdiv(d.M, 64));
    if (d.precision == GPT_BF16)
      gemm_simt_kernel<bf16_t, bf16_t><<<grid, 256, 0, s>>>(A, B, 0, e);
    else
      gemm_simt_kernel<float, float><<<grid, 256, 0, s>>>(A, B, 0, e);
    return hipGetLastError();
  }
  if (d.precision != GPT_BF16) {
    dim3 grid((unsigned)cdiv(d.N, 64), (unsigned)cdiv(d.M, 64));
    gemm_simt_kernel<float, float><<<grid, 256, 0, s>>>(A, B, d.K, e);
    return hipGetLastError();
  }
  int S = gemm_split_count(d);
  dim3 grid((unsigned)cdiv(d.N, BN), (unsigned)cdiv(d.M, BM), (unsigned)S);
  if (S == 1) {
    gemm_mfma_kernel<false><<<grid, 256, 0, s>>>(A, B, d.K, d.K, e, nullptr);
    return hipGetLastError();
  }
  const int kchunk = (int)cdiv(cdiv(d.K, S), BK) * BK;
  gemm_mfma_kernel<true><<<grid, 256, 0, s>>>(A, B, d.K, kchunk, e, (float*)d.workspace);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  long total = (long)d.M * d.N;
  unsigned blocks = (unsigned)std::min<long>(cdiv(total, 256), 4096);
  splitk_reduce_kernel<bf16_t><<<blocks, 256, 0, s>>>((const float*)d.workspace, S, e);
  return hipGetLastError();
}

}  // namespace gpt
