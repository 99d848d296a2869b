// Launchers of the HIP kernels that make up the GPT training step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gpt.h"
#include "common.h"

namespace gpt {

// Matrix products (gemm.hip).  Returns hipSuccess or the launch error;
// hipErrorInvalidValue when the descriptor breaks the stated layout rules.
// side_by_side: how many launches of this shape run at the same time on
// other streams (1 = alone); the tile plan judges how evenly a grid fills the
// CUs on that many grids (results do not depend on it).
hipError_t gemm(const gpt_gemm_desc& d, hipStream_t s, int side_by_side = 1);
// Bytes of split-K workspace gemm() may use for this shape (0 = never splits).
int64_t gemm_workspace_bytes(int M, int N, int K, int precision);
// n (<= 4) weight-gradient products with the same K in one launch (split-K
// partials in d[0].workspace, reduced per product in split order); products
// the grouped kernel cannot take, or a short workspace, run one by one.
// db (may be NULL; entries may be NULL): db[i] (+)= the column sums of the
// bf16 K-major A_i (sum over K), stored or added as the product's epilogue.
// phase: 0 = everything; 1 = the products (partials) only; 2 = the reduction
// only (after phase 1 with the same arguments; nothing when not grouped).
// sq (may be NULL): the reduction also writes, per block, the sum of squares
// of the values it stores (products and bias gradients; double, fixed order),
// gemm_group_reduce_blocks(d, n, db) entries.
hipError_t gemm_group(const gpt_gemm_desc* d, int n, hipStream_t s, float* const* db = nullptr,
                      int phase = 0, double* sq = nullptr);
constexpr int GROUP_REDUCE_MAX_BLOCKS = 8192;
// Blocks of the grouped launch's reduction (0: the products would not be
// grouped, so there is no reduction and no sum of squares).
int gemm_group_reduce_blocks(const gpt_gemm_desc* d, int n, float* const* db);
int64_t gemm_group_workspace_bytes(const int* M, const int* N, int n, int K);
// Number of K splits gemm() will use for this descriptor (1 = single kernel).
int gemm_split_count(const gpt_gemm_desc& d, int side_by_side = 1);

// Attention (attention.hip).
hipError_t attention_fwd(int prec, int B, int T, int H, int hd, int left, const void* qkv,
                         void* out, float* lse, hipStream_t s);
hipError_t attention_bwd(int prec, int B, int T, int H, int hd, int left, const void* qkv,
                         const void* out, const float* lse, const void* dout, void* dqkv,
                         float* dvec, hipStream_t s);  // dvec: 2 * B * H * T floats
bool attention_supported(int prec, int hd);
// The device address of this GPU's static attention scratch (floats) for a
// caller that needs `floats` of it; hipErrorInvalidValue beyond the maximum.
constexpr long ATTN_SCRATCH_FLOATS = 2L << 20;  // 8 MiB: B*H*T <= 1,048,576
hipError_t attention_scratch(long floats, float** out);

// Row-wise kernels (rowwise.hip).
// Ids outside [0, V) are read as 0 and mark *flag = gen; ids_out (may be
// NULL) receives the ids used.
hipError_t embed_fwd(int prec, const int32_t* idx, const float* wte, const float* wpe, int M, int T,
                     int C, int V, float* x, int32_t* ids_out, int32_t* flag, int32_t gen,
                     hipStream_t s);
// Deterministic embedding backward: dwte[v] (+)= sum of dx rows whose token is v,
// in increasing position order; dwpe[t] (+)= sum_b dx[b*T+t].
// Scratch of embed_bwd: counts/offsets [Vp], tile_sums [Vp / 1024 + 1],
// rank/perm [M], carry_first / carry_last [embed_bwd_chunks(M)][C] floats,
// flags/last_tok [chunks].
struct EmbedBwdScratch {
  int32_t* counts; int32_t* offsets; int32_t* tile_sums; int32_t* rank; int32_t* perm;
  float* carry_first; float* carry_last; int32_t* flags; int32_t* last_tok;
};
int embed_bwd_chunks(int M);
hipError_t embed_bwd(const int32_t* idx, const float* dx, int M, int T, int C, int Vp, int Tb,
                     float* dwte, int wte_accumulate, float* dwpe, int wpe_accumulate,
                     EmbedBwdScratch scr, hipStream_t s);
hipError_t layernorm_fwd(int prec, const float* x, const float* w, const float* b, int M, int C,
                         float eps, void* y, float* mean, float* rstd, hipStream_t s);
// dx = resid_in + LN'(dy); dx_act = act copy of dx; dw/db (+)= column sums.
hipError_t layernorm_bwd(int prec, const void* dy, const float* x, const float* mean,
                         const float* rstd, const float* w, const float* resid_in, int M, int C,
                         float* dx, void* dx_act, float* dw, float* db, int accumulate,
                         float* partials, hipStream_t s);
int layernorm_bwd_partial_rows(int M);
// Floats of `partials` layernorm_bwd needs.
int64_t layernorm_bwd_partial_floats(int M, int C);
// Column sums of an act-type [M, N] matrix into out[N] (overwrite or add).
hipError_t colsum(int prec, const void* x, int M, int N, float* out, int accumulate,
                  float* partials, hipStream_t s);
int colsum_partial_rows(int M);
// Floats of `partials` colsum needs.
int64_t colsum_partial_floats(int M, int N);
// Fused softmax cross-entropy on logits [M, ldz] (act type): loss_rows[m],
// logits overwritten by d(mean loss)/dlogits (0 for columns >= V).  Targets
// outside [0, V) are read as 0 and mark *flag = gen.
hipError_t cross_entropy(int prec, void* logits, int M, int V, int ldz, const int32_t* tgt,
                         float* loss_rows, int32_t* flag, int32_t gen, hipStream_t s);
bool cross_entropy_supported(int prec, int ldz);
// out = mean of loss_rows (double, fixed order); NaN when *flag == gen.
hipError_t mean_loss(const float* loss_rows, int M, float* out, const int32_t* flag, int32_t gen,
                     hipStream_t s);
// Sum of squares of x[n] (float) -> *out (double), fixed order.
hipError_t sumsq(const float* x, int64_t n, double* partials, double* out, hipStream_t s);
// Sums of squares over ranges of x: d_ranges (device) holds (begin, length,
// first block) per range, the first blocks the running sum of
// sumsq_range_blocks(length); one double per block into partials.
int sumsq_range_blocks(int64_t len);
hipError_t sumsq_ranges(const float* x, const int64_t* d_ranges, int nranges, int blocks,
                        double* partials, hipStream_t s);
// out = the sum of partials[0 .. n) in index order (double).
hipError_t sum_partials(const double* partials, int n, double* out, hipStream_t s);
hipError_t to_bf16(const float* x, int64_t n, uint16_t* y, hipStream_t s);
// Seeded initialisation: p[0 .. n) holds flat indices begin .. begin + n; the
// first n_normal get (float)(stdv * z(i)), z the Philox4x32-10 / Box-Muller
// standard normal of flat index i under `seed`, the rest 0.
hipError_t init_normal(float* p, int64_t begin, int64_t n, int64_t n_normal, double stdv,
                       uint64_t seed, hipStream_t s);
hipError_t fill_value(float* p, int64_t n, float v, hipStream_t s);

// AdamW (adamw.hip).
struct AdamScalars { float omb1, omb2, decay, step_size, sbc2, eps, scale; };
// d_scale (device, may be NULL): the gradient scale in place of sc.scale; a
// NaN there leaves p, m, v and the shadow unchanged.
// A tripped guard (common.h) leaves them unchanged too.
hipError_t adamw(int64_t n, float* p, float* m, float* v, const float* g, uint16_t* shadow,
                 AdamScalars sc, hipStream_t s, const float* d_scale = nullptr,
                 Guard guard = Guard{nullptr, 0});
// Device global-norm clip from the sum of squares at norm2: out = {norm,
// grad_scale} (doubles), scale = grad_scale as float (NaN: non-finite norm or
// a tripped guard).
hipError_t clip_scale(const double* norm2, int n_micro, double max_norm, double* out, float* scale,
                      Guard guard, hipStream_t s);
// AdamW over segments of the flat vectors in one launch.  d_seg (device):
// (begin, length, first block) per segment; lengths multiples of 4; the
// first blocks are the running sum of adamw_segment_blocks(length).
int adamw_segment_blocks(int64_t len);
hipError_t adamw_segments(const int64_t* d_seg, int nseg, int blocks, float* p, float* m,
                          float* v, const float* g, uint16_t* shadow, AdamScalars sc,
                          Guard guard, hipStream_t s);

// Generation (decode.hip).  The position of a decode step is read from
// device memory (*pos), so one captured step serves every position.
// x[b] = wte[tok[b]] + wpe[*pos]; ids outside [0, V) read row 0.
hipError_t gen_embed(const int32_t* tok, const float* wte, const float* wpe, const int32_t* pos,
                     int B, int C, int V, float* x, hipStream_t s);
hipError_t gen_set_pos(int32_t* pos, int32_t v, hipStream_t s);  // *pos = v
hipError_t gen_advance(int32_t* pos, hipStream_t s);             // *pos += 1
// One query per (sequence b, head h) at position *pos: qkv [B, 3*H*hd] (act);
// caches [B, H, Tmax, hd] (act) of this layer; row *pos of both caches is
// written from qkv; out [B, H*hd] (act).
bool attn_decode_supported(int hd);
// Few-row bf16 product of a decode step: out[b, n] = epilogue(sum_k a[b, k] W[n, k]),
// W [N, K] bf16 (K % 64 == 0).  The activation rows are a [B, K] bf16, or with x set
// LayerNorm(x) of the fp32 rows x [B, K] with ln_w / ln_b (ln_b optional) and eps.
// Epilogue STORE / RESIDUAL (out and resid float, no LayerNorm) / GELU (aux = GELU of
// the stored pre-activation), bias optional.
struct RowsLinear {
  const void* a = nullptr;
  const float* x = nullptr;
  const float* ln_w = nullptr;
  const float* ln_b = nullptr;
  float eps = 0.f;
  int B = 0, K = 0, N = 0;
  const void* W = nullptr;
  const float* bias = nullptr;
  int epi = 0;
  void* out = nullptr;
  long ldo = 0;
  const float* resid = nullptr;
  void* aux = nullptr;
  int tanh_form = 0;
};
constexpr int ROWS_LINEAR_MAX_LN_K = 1024;  // LayerNorm rows staged in LDS
hipError_t rows_linear(const RowsLinear& p, hipStream_t s);
hipError_t attn_decode(int prec, int hd, const void* qkv, void* kc, void* vc, const int32_t* pos,
                       int Tmax, int B, int H, int left, void* out, hipStream_t s);
// Per row b of logits [B, ldz] (act): token from the first V entries with
// u[b * u_stride]; written to tok[b] and, if seq, seq[b * seq_stride + seq_col].
hipError_t sample(int prec, const void* logits, long ldz, int B, int V, float temperature,
                  int top_k, const float* u, long u_stride, int32_t* tok, int32_t* seq,
                  long seq_stride, int seq_col, hipStream_t s);
hipError_t gather_column(const int32_t* seq, long stride, int col, int B, int32_t* tok,
                         hipStream_t s);
hipError_t copy_prompt(const int32_t* prompt, int T0, int Ltot, int B, int32_t* out,
                       hipStream_t s);

// Muon for one kind of block matrix across the layers (muon.hip).  Matrix l
// (l < count) of shape [rows, cols] sits at element offset l * ls of the
// parameter, gradient, momentum (buf) and second-moment (v, first max(rows,
// cols) entries used) arrays, all given at layer 0.  `shadow` (bf16 copy of
// p, bf16 mode) may be NULL.
struct MuonGroup {
  const float* g; float* buf; float* v; float* p; uint16_t* shadow;
  long ls; int rows, cols, count;
};
struct MuonScalars {
  float grad_scale, omm, mu, omb2, eps, lr, lrwd;  // omm = 1 - mu, omb2 = 1 - beta2, lrwd = lr * wd
  float a, b, c;                                  // Newton-Schulz polynomial
  int ns_steps;
};
constexpr int MUON_PREP_BLOCKS = 64;  // sum-of-squares partials per matrix
// Workspace bytes muon_matrices needs for `count` matrices of [rows, cols].
int64_t muon_workspace_bytes(int rows, int cols, int count, int prec);
// A tripped guard leaves the parameters, momentum and second moment unchanged.
hipError_t muon_matrices(const MuonGroup& g, const MuonScalars& sc, int prec, void* workspace,
                         Guard guard, hipStream_t s);

}  // namespace gpt
