// Muon for the per-layer Linear weights (nanochat "Optimierungsstrategien Muon
// und AdamW": Muon orthogonalizes the update of every 2-D attention / MLP
// matrix by a Newton-Schulz iteration; a factored second moment and a
// cautious update follow).  The element-wise stages live here; the iteration's
// matrix products run through the batched MFMA GEMM (one launch covers the
// same matrix of every layer).
//
// Stages per matrix W [r, c] with gradient G (one launch each, grid.y = layer):
//   prep    g = G * grad_scale; buf += (1-mu)(g - buf); u = g + mu (buf - g);
//           X = act(u); per-block sums of X^2 (double)
//   norm    den = ||X||_F * 1.01 + 1e-6 (bf16 mode: each step rounded to bf16,
//           as the page's bf16 tensors round)
//   scale   X = act(X / den)
//   (5 x: A = Gram(X); B = c A A + b A; X = a X + X B  or  B X, wide)
//   stats   s_i = mean of X^2 over the shorter dimension, i along the longer
//   second  v_i += (1-beta2)(s_i - v_i); d_i = sqrt(v_i) + eps; the factor
//           f = ||X|| / ||X / d|| restores the Frobenius norm; r_i = f / d_i
//   update  y = X r_i; p -= lr y + lr wd p [y p >= 0]; bf16 copy of p
//
// Compiled with -ffp-contract=off so the momentum matches the same float32
// operation sequence anywhere else bit for bit.

#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <cstring>
#include <utility>

namespace gpt {

namespace {

constexpr int MU_THREADS = 256;

__device__ __forceinline__ double block_sum_d(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int w = MU_THREADS / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

template <typename ActT>
__global__ void __launch_bounds__(MU_THREADS) muon_prep_kernel(
    const float* __restrict__ g, float* __restrict__ buf, long ls, long rc, float scale,
    float omm, float mu, ActT* __restrict__ X, int chunk, double* __restrict__ part, Guard guard) {
  __shared__ double red[MU_THREADS];
  const bool frozen = guard_tripped(guard);  // momentum left unchanged
  const int l = blockIdx.y;
  const float* gl = g + l * ls;
  float* bl = buf + l * ls;
  ActT* xl = X + l * rc;
  const long b = (long)blockIdx.x * chunk, e = min(rc, b + chunk);
  float ss = 0.f;
  for (long i = b + threadIdx.x * 4; i < e; i += MU_THREADS * 4) {  // rc, chunk: multiples of 4
    const float4 g4 = *(const float4*)(gl + i);
    float4 m4 = *(float4*)(bl + i);
    float gv[4] = {g4.x, g4.y, g4.z, g4.w}, mv[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float gs = gv[k] * scale;
      mv[k] = mv[k] + omm * (gs - mv[k]);
      const float u = gs + mu * (mv[k] - gs);
      Act<ActT>::store(xl, i + k, u);
      const float x = Act<ActT>::load(xl, i + k);
      ss += x * x;
    }
    if (!frozen) *(float4*)(bl + i) = make_float4(mv[0], mv[1], mv[2], mv[3]);
  }
  const double t = block_sum_d((double)ss, red);
  if (threadIdx.x == 0) part[(long)l * gridDim.x + blockIdx.x] = t;
}

template <bool BF16>
__global__ void __launch_bounds__(MU_THREADS) muon_norm_kernel(const double* __restrict__ part,
                                                              int nb, float* __restrict__ den) {
  __shared__ double red[MU_THREADS];
  const int l = blockIdx.x;
  double s = 0.0;
  for (int i = threadIdx.x; i < nb; i += MU_THREADS) s += part[(long)l * nb + i];
  s = block_sum_d(s, red);
  if (threadIdx.x == 0) {
    const double n = sqrt(s);
    if (BF16) {
      const float nb16 = bf2f(f2bf((float)n));
      const float t = bf2f(f2bf(nb16 * 1.01f));
      den[l] = bf2f(f2bf(t + 1e-6f));
    } else {
      den[l] = (float)(n * 1.01 + 1e-6);
    }
  }
}

template <typename ActT>
__global__ void __launch_bounds__(MU_THREADS) muon_scale_kernel(ActT* __restrict__ X, long rc,
                                                               const float* __restrict__ den) {
  const int l = blockIdx.y;
  ActT* xl = X + l * rc;
  const float d = den[l];
  for (long i = (long)blockIdx.x * MU_THREADS + threadIdx.x; i < rc;
       i += (long)gridDim.x * MU_THREADS)
    Act<ActT>::store(xl, i, __fdiv_rn(Act<ActT>::load(xl, i), d));
}

// Tall matrices (r > c): one wave per row, s_i over the c columns.
template <typename ActT>
__global__ void __launch_bounds__(MU_THREADS) muon_row_stats_kernel(const ActT* __restrict__ X,
                                                                   int r, int c,
                                                                   float* __restrict__ s) {
  const int l = blockIdx.y;
  const int row = blockIdx.x * (MU_THREADS / 64) + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= r) return;
  const ActT* x = X + ((long)l * r + row) * c;
  float a = 0.f;
  for (int j = lane; j < c; j += 64) {
    const float v = Act<ActT>::load(x, j);
    a += v * v;
  }
  a = warp_sum(a);
  if (lane == 0) s[(long)l * r + row] = a / (float)c;
}

// Wide and square matrices (r <= c): a block takes 64 columns; its 4 waves
// sum every 4th row (one 64-column row segment per wave and step), then the
// four partial sums are added in a fixed order.
template <typename ActT>
__global__ void __launch_bounds__(MU_THREADS) muon_col_stats_kernel(const ActT* __restrict__ X,
                                                                   int r, int c,
                                                                   float* __restrict__ s) {
  __shared__ float part[MU_THREADS / 64][64];
  const int l = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + lane;
  float a = 0.f;
  if (col < c) {
    const ActT* x = X + (long)l * r * c + col;
    for (int i = wave; i < r; i += MU_THREADS / 64) {
      const float v = Act<ActT>::load(x, (long)i * c);
      a += v * v;
    }
  }
  part[wave][lane] = a;
  __syncthreads();
  if (wave == 0 && col < c) {
    float t = part[0][lane];
    for (int w = 1; w < MU_THREADS / 64; ++w) t += part[w][lane];
    s[(long)l * c + col] = t / (float)r;
  }
}

// One block per matrix: the running second moment (first n_long entries of
// the matrix's v slot) and the per-row (per-column) factors r_i.
__global__ void __launch_bounds__(MU_THREADS) muon_second_kernel(
    const float* __restrict__ s, float* __restrict__ v, long ls, int n_long, int n_short,
    float omb2, float eps, float* __restrict__ rfac, Guard guard) {
  __shared__ double red[MU_THREADS];
  if (guard_tripped(guard)) return;  // second moment left unchanged (no update follows)
  const int l = blockIdx.x;
  const float* sl = s + (long)l * n_long;
  float* vl = v + l * ls;
  float* rl = rfac + (long)l * n_long;
  double x2 = 0.0, y2 = 0.0;
  for (int i = threadIdx.x; i < n_long; i += MU_THREADS) {
    const float si = sl[i];
    const float vi = vl[i] + omb2 * (si - vl[i]);
    vl[i] = vi;
    const double d = (double)sqrtf(vi) + (double)eps;
    x2 += (double)si;
    y2 += (double)si / (d * d);
  }
  x2 = block_sum_d(x2, red);
  y2 = block_sum_d(y2, red);
  const double f = y2 > 0.0 ? sqrt(x2 / y2) : 1.0;  // n_short cancels in the ratio
  (void)n_short;
  for (int i = threadIdx.x; i < n_long; i += MU_THREADS) {
    const double d = (double)sqrtf(vl[i]) + (double)eps;
    rl[i] = (float)(f / d);
  }
}

template <typename ActT>
__global__ void __launch_bounds__(MU_THREADS) muon_update_kernel(
    float* __restrict__ p, long ls, const ActT* __restrict__ X, int r, int c, int tall,
    const float* __restrict__ rfac, float lr, float lrwd, bf16_t* __restrict__ shadow,
    Guard guard) {
  if (guard_tripped(guard)) return;
  const int l = blockIdx.y;
  const long rc = (long)r * c;
  float* pl = p + l * ls;
  bf16_t* sh = shadow ? shadow + l * ls : nullptr;
  const ActT* xl = X + l * rc;
  const float* rl = rfac + (long)l * (tall ? r : c);
  // 4 consecutive elements of one row per thread (c % 4 == 0).
  for (long i = ((long)blockIdx.x * MU_THREADS + threadIdx.x) * 4; i < rc;
       i += (long)gridDim.x * MU_THREADS * 4) {
    const int row = (int)(i / c), col = (int)(i - (long)row * c);
    float4 p4 = *(const float4*)(pl + i);
    float pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float y = Act<ActT>::load(xl, i + k) * rl[tall ? row : col + k];
      const float dec = (y * pv[k] >= 0.f) ? lrwd * pv[k] : 0.f;
      pv[k] = pv[k] - (lr * y + dec);
    }
    *(float4*)(pl + i) = make_float4(pv[0], pv[1], pv[2], pv[3]);
    if (sh) *(uint2*)(sh + i) = make_uint2(pack_bf2(pv[0], pv[1]), pack_bf2(pv[2], pv[3]));
  }
}

}  // namespace

int64_t muon_workspace_bytes(int r, int c, int L, int prec) {
  const int64_t act = prec == GPT_BF16 ? 2 : 4;
  const int64_t sq = (int64_t)std::min(r, c) * std::min(r, c);
  const int64_t nl = std::max(r, c);
  auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  return 2 * al((int64_t)L * r * c * act) + 2 * al(L * sq * act) +
         al((int64_t)L * MUON_PREP_BLOCKS * 8) + al(L * 4) + 2 * al(L * nl * 4);
}

hipError_t muon_matrices(const MuonGroup& gp, const MuonScalars& sc, int prec, void* ws,
                         Guard guard, hipStream_t s) {
  const int r = gp.rows, c = gp.cols, L = gp.count;
  if (L <= 0) return hipSuccess;
  const bool bf16 = prec == GPT_BF16;
  const int64_t act = bf16 ? 2 : 4;
  const long rc = (long)r * c;
  const int sdim = std::min(r, c), nl = std::max(r, c);
  const bool tall = r > c;
  auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  char* w = (char*)ws;
  void* X0 = w;                       w += al((int64_t)L * rc * act);
  void* X1 = w;                       w += al((int64_t)L * rc * act);
  void* Am = w;                       w += al((int64_t)L * sdim * sdim * act);
  void* Bm = w;                       w += al((int64_t)L * sdim * sdim * act);
  double* part = (double*)w;          w += al((int64_t)L * MUON_PREP_BLOCKS * 8);
  float* den = (float*)w;             w += al((int64_t)L * 4);
  float* st = (float*)w;              w += al((int64_t)L * nl * 4);
  float* rfac = (float*)w;

  // prep: momentum, act copy, sums of squares
  const int chunk = (int)((rc + MUON_PREP_BLOCKS - 1) / MUON_PREP_BLOCKS + 3) / 4 * 4;
  const int nb = (int)((rc + chunk - 1) / chunk);
  dim3 gprep((unsigned)nb, (unsigned)L);
  if (bf16)
    muon_prep_kernel<bf16_t><<<gprep, MU_THREADS, 0, s>>>(gp.g, gp.buf, gp.ls, rc, sc.grad_scale,
                                                          sc.omm, sc.mu, (bf16_t*)X0, chunk, part,
                                                          guard);
  else
    muon_prep_kernel<float><<<gprep, MU_THREADS, 0, s>>>(gp.g, gp.buf, gp.ls, rc, sc.grad_scale,
                                                         sc.omm, sc.mu, (float*)X0, chunk, part,
                                                         guard);
  if (bf16)
    muon_norm_kernel<true><<<L, MU_THREADS, 0, s>>>(part, nb, den);
  else
    muon_norm_kernel<false><<<L, MU_THREADS, 0, s>>>(part, nb, den);
  const unsigned eb = (unsigned)std::min<long>((rc + MU_THREADS - 1) / MU_THREADS, 1024);
  if (bf16)
    muon_scale_kernel<bf16_t><<<dim3(eb, L), MU_THREADS, 0, s>>>((bf16_t*)X0, rc, den);
  else
    muon_scale_kernel<float><<<dim3(eb, L), MU_THREADS, 0, s>>>((float*)X0, rc, den);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // Newton-Schulz iterations, batched over the layers.
  gpt_gemm_desc d;
  auto base = [&](int M, int N, int K) {
    std::memset(&d, 0, sizeof(d));
    d.precision = prec;
    d.M = M; d.N = N; d.K = K;
    d.batch = L;
  };
  void* X = X0;
  void* Xn = X1;
  for (int it = 0; it < sc.ns_steps; ++it) {
    // A = X^T X (tall) or X X^T (wide), [sdim, sdim]
    base(sdim, sdim, tall ? r : c);
    if (tall) {
      d.A = X; d.lda = c; d.a_trans = 1; d.a_rows = c; d.a_kvalid = r;
      d.B = X; d.ldb = c; d.b_trans = 1; d.b_rows = c; d.b_kvalid = r;
    } else {
      d.A = X; d.lda = c; d.a_trans = 0; d.a_rows = r; d.a_kvalid = c;
      d.B = X; d.ldb = c; d.b_trans = 0; d.b_rows = r; d.b_kvalid = c;
    }
    d.epilogue = GPT_EPI_STORE;
    d.out = Am; d.ldo = sdim;
    d.stride_a = d.stride_b = rc * act;
    d.stride_out = (int64_t)sdim * sdim * act;
    if ((err = gemm(d, s)) != hipSuccess) return err;
    // B = c A A + b A  (A is symmetric: its rows serve as the second operand)
    base(sdim, sdim, sdim);
    d.A = Am; d.lda = sdim; d.a_trans = 0; d.a_rows = sdim; d.a_kvalid = sdim;
    d.B = Am; d.ldb = sdim; d.b_trans = 0; d.b_rows = sdim; d.b_kvalid = sdim;
    d.epilogue = GPT_EPI_AXPBY; d.alpha = sc.c; d.beta = sc.b;
    d.aux = Am; d.ldaux = sdim;
    d.out = Bm; d.ldo = sdim;
    d.stride_a = d.stride_b = d.stride_aux = d.stride_out = (int64_t)sdim * sdim * act;
    if ((err = gemm(d, s)) != hipSuccess) return err;
    // X' = a X + X B (tall) or a X + B X (wide)
    base(r, c, sdim);
    if (tall) {
      d.A = X; d.lda = c; d.a_trans = 0; d.a_rows = r; d.a_kvalid = c;
      d.B = Bm; d.ldb = c; d.b_trans = 0; d.b_rows = c; d.b_kvalid = c;
      d.stride_a = rc * act;
      d.stride_b = (int64_t)sdim * sdim * act;
    } else {
      d.A = Bm; d.lda = r; d.a_trans = 0; d.a_rows = r; d.a_kvalid = r;
      d.B = X; d.ldb = c; d.b_trans = 1; d.b_rows = c; d.b_kvalid = r;
      d.stride_a = (int64_t)sdim * sdim * act;
      d.stride_b = rc * act;
    }
    d.epilogue = GPT_EPI_AXPBY; d.alpha = 1.f; d.beta = sc.a;
    d.aux = X; d.ldaux = c; d.stride_aux = rc * act;
    d.out = Xn; d.ldo = c; d.stride_out = rc * act;
    if ((err = gemm(d, s)) != hipSuccess) return err;
    std::swap(X, Xn);
  }

  // Factored second moment and the cautious update.
  if (tall) {
    dim3 gs((unsigned)((r + MU_THREADS / 64 - 1) / (MU_THREADS / 64)), (unsigned)L);
    if (bf16)
      muon_row_stats_kernel<bf16_t><<<gs, MU_THREADS, 0, s>>>((const bf16_t*)X, r, c, st);
    else
      muon_row_stats_kernel<float><<<gs, MU_THREADS, 0, s>>>((const float*)X, r, c, st);
  } else {
    dim3 gs((unsigned)((c + 63) / 64), (unsigned)L);
    if (bf16)
      muon_col_stats_kernel<bf16_t><<<gs, MU_THREADS, 0, s>>>((const bf16_t*)X, r, c, st);
    else
      muon_col_stats_kernel<float><<<gs, MU_THREADS, 0, s>>>((const float*)X, r, c, st);
  }
  muon_second_kernel<<<L, MU_THREADS, 0, s>>>(st, gp.v, gp.ls, nl, sdim, sc.omb2, sc.eps, rfac,
                                              guard);
  if (bf16)
    muon_update_kernel<bf16_t><<<dim3(eb, L), MU_THREADS, 0, s>>>(
        gp.p, gp.ls, (const bf16_t*)X, r, c, tall, rfac, sc.lr, sc.lrwd, (bf16_t*)gp.shadow,
        guard);
  else
    muon_update_kernel<float><<<dim3(eb, L), MU_THREADS, 0, s>>>(
        gp.p, gp.ls, (const float*)X, r, c, tall, rfac, sc.lr, sc.lrwd, (bf16_t*)gp.shadow,
        guard);
  return hipGetLastError();
}

}  // namespace gpt
