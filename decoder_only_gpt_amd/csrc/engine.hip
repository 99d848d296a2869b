// Host side of the GPT step: configuration checks, the device-arena plan, the
// launch sequences of forward / backward / norm / AdamW, the call-order state
// machine and the extern "C" entry points declared in include/gpt.h.
//
// Call order follows the training loop of the NiNo README ("usage": model
// output -> cross_entropy -> backward -> step -> zero_grad) and the
// flattened-parameter model adapter of the Panthalia plugin page
// ("Components"): one flat float32 vector of parameters, with gradients and
// both AdamW moments in the same layout.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "../../include/gpt.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      return fail(GPT_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));         \
  } while (0)

constexpr int64_t ALIGN = 256;
int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct LayerOff {  // element offsets into the flat parameter vector (-1 = absent)
  int64_t ln1w, ln1b, qkvw, qkvb, projw, projb, ln2w, ln2b, fcw, fcb, fcpw, fcpb;
};

struct ParamLayout {
  int64_t wte, wpe, lnfw, lnfb, lmw, n;
  std::vector<LayerOff> layer;
};

ParamLayout param_layout(const gpt_config& c) {
  ParamLayout p;
  const int64_t C = c.n_embd, F = c.mlp_hidden;
  int64_t o = 0;
  auto take = [&](int64_t n) { int64_t r = o; o += n; return r; };
  p.wte = take((int64_t)c.padded_vocab * C);
  p.wpe = take((int64_t)c.block_size * C);
  for (int l = 0; l < c.n_layer; ++l) {
    LayerOff L;
    L.ln1w = take(C);
    L.ln1b = c.bias ? take(C) : -1;
    L.qkvw = take(3 * C * C);
    L.qkvb = c.bias ? take(3 * C) : -1;
    L.projw = take(C * C);
    L.projb = c.bias ? take(C) : -1;
    L.ln2w = take(C);
    L.ln2b = c.bias ? take(C) : -1;
    L.fcw = take(F * C);
    L.fcb = c.bias ? take(F) : -1;
    L.fcpw = take(C * F);
    L.fcpb = c.bias ? take(C) : -1;
    p.layer.push_back(L);
  }
  p.lnfw = take(C);
  p.lnfb = c.bias ? take(C) : -1;
  p.lmw = c.tied_lm_head ? p.wte : take((int64_t)c.padded_vocab * C);
  p.n = o;
  return p;
}

// The ranges of the flat vector whose gradients the grouped weight-gradient
// reductions do not write (embeddings, the LayerNorm parameters of every
// block, the final LayerNorm and an untied head): the gradient norm sums them
// separately and takes the blocks' matrices and biases from those reductions.
std::vector<std::pair<int64_t, int64_t>> norm_ranges(const gpt_config& c, const ParamLayout& p) {
  std::vector<std::pair<int64_t, int64_t>> r;
  auto add = [&](int64_t b, int64_t e) { if (e > b) r.push_back({b, e - b}); };
  add(0, c.n_layer > 0 ? p.layer[0].ln1w : p.lnfw);
  for (const LayerOff& L : p.layer) {
    add(L.ln1w, L.qkvw);
    add(L.ln2w, L.fcw);
  }
  add(p.lnfw, p.n);
  return r;
}

int64_t n_matmul(const gpt_config& c) {
  const int64_t C = c.n_embd, F = c.mlp_hidden;
  return (int64_t)c.n_layer * (3 * C * C + C * C + 2 * F * C) + (int64_t)c.padded_vocab * C;
}

double flops_per_token(const gpt_config& c, int T) {
  const int64_t hd = c.n_embd / c.n_head;
  double attn = 0;
  for (int l = 0; l < c.n_layer; ++l) {
    int w = c.window_left[l];
    int64_t eff = w < 0 ? T : std::min<int64_t>(w, T);
    attn += 12.0 * c.n_head * hd * eff;
  }
  return 6.0 * (double)n_matmul(c) + attn;
}

int check_config(const gpt_config* c, int B, int T) {
  if (!c) return fail(GPT_E_INVALID, "config is NULL");
  if (c->vocab_size < 1 || c->padded_vocab < c->vocab_size)
    return fail(GPT_E_INVALID, "need 1 <= vocab_size <= padded_vocab");
  if (c->block_size < 1) return fail(GPT_E_INVALID, "block_size < 1");
  if (c->n_layer < 1 || c->n_layer > GPT_MAX_LAYERS) return fail(GPT_E_INVALID, "bad n_layer");
  if (c->n_head < 1 || c->n_embd < 1 || c->n_embd % c->n_head)
    return fail(GPT_E_INVALID, "n_embd must be a positive multiple of n_head");
  if (c->n_embd % 64 || c->mlp_hidden < 64 || c->mlp_hidden % 64)
    return fail(GPT_E_INVALID, "n_embd and mlp_hidden must be multiples of 64");
  if (c->precision != GPT_FP32 && c->precision != GPT_BF16)
    return fail(GPT_E_INVALID, "precision must be 0 (fp32) or 1 (bf16)");
  if (!(c->ln_eps > 0.f)) return fail(GPT_E_INVALID, "ln_eps must be > 0");
  if (B < 1 || T < 1 || T > c->block_size)
    return fail(GPT_E_INVALID, "need B >= 1 and 1 <= T <= block_size");
  if ((int64_t)B * T > (1 << 26)) return fail(GPT_E_UNSUPPORTED, "B*T too large");
  if (c->n_embd > 2048) return fail(GPT_E_UNSUPPORTED, "n_embd > 2048");
  const int hd = c->n_embd / c->n_head;
  if (!gpt::attention_supported(c->precision, hd))
    return fail(GPT_E_UNSUPPORTED, "head_dim " + std::to_string(hd) +
                                       " not supported (bf16: 32/64/128; fp32: <= 128)");
  const int Vq = (int)align_up(c->padded_vocab, 64);
  if (!gpt::cross_entropy_supported(c->precision, Vq))
    return fail(GPT_E_UNSUPPORTED, "padded vocabulary too large for the fused cross-entropy");
  return GPT_OK;
}

// Depth of the rings of gradient buffers shared by the two backward streams.
constexpr int NGB = 6;

// Byte offsets of every region of the arena.
struct Arena {
  int64_t params, grads, adam_m, adam_v, shadow;
  int64_t X, ln_mean, ln_rstd;
  std::vector<int64_t> a1, qkv, att, lse, a2, u, g;
  int64_t xf, logits, loss_rows, loss, gres[2], gact[NGB], dC, dC2, dF[NGB], dqkv[NGB], dvec;
  int64_t gemm_ws, gemm_ws_bytes, cs_part, ln_part, n_part, n_rng, norm2, clip, muon_ws, adam_seg;
  int64_t e_counts, e_offsets, e_tile_sums, e_rank, e_perm, e_carry_first, e_carry_last, e_flags,
      e_last_tok;
  int64_t ids, id_flag;  // token ids the forward used; forward count of the last bad id
  int64_t state_end, total;
};

Arena plan_arena(const gpt_config& c, int B, int T) {
  Arena a;
  const int64_t M = (int64_t)B * T, C = c.n_embd, F = c.mlp_hidden, L = c.n_layer;
  const int64_t H = c.n_head, Vp = c.padded_vocab, Vq = align_up(Vp, 64);
  const int64_t act = c.precision == GPT_BF16 ? 2 : 4;
  const int64_t N = param_layout(c).n;
  int64_t o = 0;
  auto take = [&](int64_t bytes) { int64_t r = o; o = align_up(o + bytes, ALIGN); return r; };
  a.params = take(N * 4);
  a.grads = take(N * 4);
  a.adam_m = take(N * 4);
  a.adam_v = take(N * 4);
  a.shadow = c.precision == GPT_BF16 ? take(N * 2) : -1;
  a.state_end = o;
  a.X = take((2 * L + 1) * M * C * 4);
  a.ln_mean = take((2 * L + 1) * M * 4);
  a.ln_rstd = take((2 * L + 1) * M * 4);
  for (int64_t l = 0; l < L; ++l) {
    a.a1.push_back(take(M * C * act));
    a.qkv.push_back(take(M * 3 * C * act));
    a.att.push_back(take(M * C * act));
    a.lse.push_back(take(M * H * 4));
    a.a2.push_back(take(M * C * act));
    a.u.push_back(take(M * F * act));
    a.g.push_back(c.recompute_gelu ? -1 : take(M * F * act));
  }
  a.xf = take(M * C * act);
  a.logits = take(M * Vq * act);
  a.loss_rows = take(M * 4);
  a.loss = take(16);
  a.gres[0] = take(M * C * 4);
  a.gres[1] = take(M * C * 4);
  // Gradients the weight-gradient branch reads live in rings of NGB buffers,
  // so the main chain can run ahead of the side stream by a few layers.
  for (int i = 0; i < NGB; ++i) a.gact[i] = take(M * C * act);
  a.dC = take(M * C * act);
  a.dC2 = take(M * C * act);
  for (int i = 0; i < NGB; ++i) a.dF[i] = take(M * F * act);
  for (int i = 0; i < NGB; ++i) a.dqkv[i] = take(M * 3 * C * act);
  a.dvec = take(2 * M * H * 4);  // D, then the log-sum-exp in log2 units
  int64_t ws = 0;
  auto ws_need = [&](int64_t m, int64_t n, int64_t k) {
    ws = std::max<int64_t>(ws, gpt::gemm_workspace_bytes((int)m, (int)n, (int)k, c.precision));
  };
  ws_need(3 * C, C, M);
  ws_need(C, C, M);
  ws_need(F, C, M);
  ws_need(C, F, M);
  ws_need(Vp, C, M);
  ws_need(M, C, Vq);  // the vocabulary projection's input gradient
  {  // a block's four weight gradients as one grouped launch
    const int gm[4] = {(int)C, (int)F, (int)C, (int)(3 * C)}, gn[4] = {(int)F, (int)C, (int)C, (int)C};
    ws = std::max<int64_t>(ws, gpt::gemm_group_workspace_bytes(gm, gn, 4, (int)M));
  }
  a.gemm_ws_bytes = ws;
  a.gemm_ws = take(std::max<int64_t>(ws, 16));
  a.cs_part = take(gpt::colsum_partial_floats((int)M, (int)std::max(3 * C, F)) * 4 + 16);
  a.ln_part = take(gpt::layernorm_bwd_partial_floats((int)M, (int)C) * 4 + 16);
  a.e_counts = take(Vp * 4);
  a.e_offsets = take(Vp * 4);
  a.e_tile_sums = take((Vp / 1024 + 1) * 4);
  a.e_rank = take(M * 4);
  a.e_perm = take(M * 4);
  const int64_t nch = gpt::embed_bwd_chunks((int)M);
  a.e_carry_first = take(nch * C * 4);
  a.e_carry_last = take(nch * C * 4);
  a.e_flags = take(nch * 4);
  a.e_last_tok = take(nch * 4);
  a.ids = take(M * 4);
  a.id_flag = take(16);
  {  // norm partials: one full pass, or the blocks' reductions plus the other ranges
    const std::vector<std::pair<int64_t, int64_t>> nr = norm_ranges(c, param_layout(c));
    int64_t nb = L * gpt::GROUP_REDUCE_MAX_BLOCKS;
    for (const auto& x : nr) nb += gpt::sumsq_range_blocks(x.second);
    a.n_part = take(std::max<int64_t>(1024, nb) * 8);
    a.n_rng = take((int64_t)nr.size() * 3 * 8 + 8);
  }
  a.norm2 = take(16);
  a.clip = take(32);  // device clip: {norm, grad_scale} doubles, then grad_scale as float
  // Muon working set, sized for the largest kind of block matrix (one kind at a time).
  int64_t mw = 0;
  for (auto rc : {std::pair<int64_t, int64_t>{3 * C, C}, {C, C}, {F, C}, {C, F}})
    mw = std::max<int64_t>(mw, gpt::muon_workspace_bytes((int)rc.first, (int)rc.second, (int)L,
                                                         c.precision));
  a.muon_ws = take(mw);
  a.adam_seg = take((4 * L + 4) * 3 * 8);  // AdamW segments of the Muon step
  a.total = o;
  return a;
}

}  // namespace

struct gpt_model {
  gpt_config cfg;
  int B, T;
  int64_t M, C, F, H, hd, Vp, Vq, N;
  bool bf16;
  ParamLayout pl;
  Arena ar;
  char* base;
  int state;  // 0 idle, 1 forward with targets done, 2 backward done
  // kernel timing (gpt_profile_begin / gpt_profile_end)
  struct Rec { int kind, site; double flops, bytes; hipEvent_t a, b; };
  bool prof_on = false;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  std::vector<Rec> recs;
  hipEvent_t next_event() {
    if (ev_used == ev_pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      ev_pool.push_back(e);
    }
    return ev_pool[ev_used++];
  }
  bool loss_valid;
  // Token-id guard: forwards are counted from 1 (gen); a forward that meets an
  // id or target outside [0, vocab_size) writes its count to the id flag.
  // upd_gen is the count at the last parameter update, so a flag > upd_gen
  // means a bad id since then.
  int32_t gen = 0, upd_gen = 0;
  int32_t* id_flag() const { return at<int32_t>(ar.id_flag); }
  gpt::Guard guard() const { return gpt::Guard{id_flag(), upd_gen + 1}; }
  // Weight-gradient branch of the backward: a second stream (default
  // priority) and the events that order it against the main chain.
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr, ev_lmdw = nullptr;
  // Further batch chains of the forward's blocks (default priority).  Two
  // chains: four made the GPT-2 124M step slower (19.2 against 18.15 ms).
  static constexpr int FWD_CHAINS = 2;
  hipStream_t fwdc[FWD_CHAINS - 1] = {};
  hipEvent_t ev_ffork = nullptr, ev_fjoin[FWD_CHAINS - 1] = {};
  hipEvent_t ev_buf[3 * NGB] = {};  // block l's grouped weight gradients done (index l % 18)
  // AdamW runs on the side stream in parameter groups (embeddings, each layer,
  // the final LayerNorm and untied head); the next forward waits per group.
  std::vector<hipEvent_t> ev_adam;
  bool adam_pending = false;
  // Gradient norm from the backward's partial sums of squares (the blocks'
  // weight-gradient reductions, then the remaining ranges): valid until the
  // gradients are rewritten otherwise.
  std::vector<int64_t> norm_rng;  // (begin, length, first block) per range
  int norm_rng_blocks = 0;
  bool norm_parts = false;
  int64_t norm_part_count = 0;
  // The runs of the flat vector outside the Muon matrices (AdamW in the
  // Muon step): (begin, length, first block) triples, also on the device.
  std::vector<int64_t> adam_seg;
  int adam_seg_blocks = 0;

  template <typename T_> T_* at(int64_t off) const { return off < 0 ? nullptr : (T_*)(base + off); }
  float* P(int64_t e) const { return e < 0 ? nullptr : at<float>(ar.params) + e; }
  float* G(int64_t e) const { return e < 0 ? nullptr : at<float>(ar.grads) + e; }
  // Weight operand of a matrix product: bf16 copy in bf16 mode, master otherwise.
  const void* W(int64_t e) const {
    return bf16 ? (const void*)(at<uint16_t>(ar.shadow) + e) : (const void*)(P(e));
  }
  float* X(int64_t i) const { return at<float>(ar.X) + i * M * C; }
  float* mean(int64_t i) const { return at<float>(ar.ln_mean) + i * M; }
  float* rstd(int64_t i) const { return at<float>(ar.ln_rstd) + i * M; }
  int prec() const { return cfg.precision; }
};

namespace {

gpt_gemm_desc gemm_desc(const gpt_model* m) {
  gpt_gemm_desc d;
  std::memset(&d, 0, sizeof(d));
  d.precision = m->cfg.precision;
  d.gelu_tanh = m->cfg.gelu_tanh;
  d.workspace = m->at<void>(m->ar.gemm_ws);
  d.workspace_bytes = m->ar.gemm_ws_bytes;
  return d;
}

// y[M, N] = x[M, K] . W[N, K]^T  (x row-major, W the [out, in] weight).
gpt_gemm_desc linear_fwd(const gpt_model* m, const void* x, int64_t K, int64_t w_off, int64_t N,
                         int64_t w_rows) {
  gpt_gemm_desc d = gemm_desc(m);
  d.M = (int)m->M; d.N = (int)N; d.K = (int)K;
  d.A = x; d.lda = K; d.a_trans = 0; d.a_rows = (int)m->M; d.a_kvalid = (int)K;
  d.B = m->W(w_off); d.ldb = K; d.b_trans = 0; d.b_rows = (int)w_rows; d.b_kvalid = (int)K;
  return d;
}

// dx[M, K] = dy[M, N] . W[N, K]  (reduction over N).
gpt_gemm_desc linear_dx(const gpt_model* m, const void* dy, int64_t N, int64_t w_off, int64_t K,
                        int64_t ldy, int64_t w_rows) {
  gpt_gemm_desc d = gemm_desc(m);
  d.M = (int)m->M; d.N = (int)K; d.K = (int)N;
  d.A = dy; d.lda = ldy; d.a_trans = 0; d.a_rows = (int)m->M; d.a_kvalid = (int)N;
  d.B = m->W(w_off); d.ldb = K; d.b_trans = 1; d.b_rows = (int)K; d.b_kvalid = (int)w_rows;
  // Input gradients run on the main stream while the side stream's weight
  // gradients own the split-K workspace: they never split (the vocabulary
  // projection's, issued before the side stream starts, gets it back).
  d.workspace = nullptr;
  d.workspace_bytes = 0;
  return d;
}

// dW[N, K] (+)= dy[M, N]^T . x[M, K]  (reduction over the M tokens).
gpt_gemm_desc linear_dw(const gpt_model* m, const void* dy, int64_t N, int64_t ldy, const void* x,
                        int64_t K, int64_t w_off, int64_t w_rows, int accumulate) {
  gpt_gemm_desc d = gemm_desc(m);
  d.M = (int)w_rows; d.N = (int)K; d.K = (int)m->M;
  d.A = dy; d.lda = ldy; d.a_trans = 1; d.a_rows = (int)w_rows; d.a_kvalid = (int)m->M;
  d.B = x; d.ldb = K; d.b_trans = 1; d.b_rows = (int)K; d.b_kvalid = (int)m->M;
  d.epilogue = accumulate ? GPT_EPI_F32_ACCUM : GPT_EPI_F32;
  d.out = m->G(w_off); d.ldo = K;
  (void)N;
  return d;
}

// Launch `f` (returns hipError_t); inside a profile window bracket it with events.
template <typename Fn>
int launch(gpt_model* m, hipStream_t s, int kind, int site, double flops, double bytes,
           const char* what, Fn f) {
  hipEvent_t a = nullptr;
  if (m->prof_on && (a = m->next_event()) != nullptr) (void)hipEventRecord(a, s);
  hipError_t e = f();
  if (e != hipSuccess) return fail(GPT_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  if (a) {
    hipEvent_t b = m->next_event();
    if (b) {
      (void)hipEventRecord(b, s);
      m->recs.push_back({kind, site, flops, bytes, a, b});
    }
  }
  return GPT_OK;
}

#define LAUNCH(kind, site, flops, bytes, expr)                                    \
  do {                                                                            \
    int rc_ = launch(m, s, kind, site, (double)(flops), (double)(bytes), #expr,   \
                     [&]() { return (expr); });                                   \
    if (rc_ != GPT_OK) return rc_;                                                \
  } while (0)

// side_by_side: launches of this shape running at the same time (batch chains).
int run_gemm(gpt_model* m, hipStream_t s, const gpt_gemm_desc& d, int site,
             int side_by_side = 1) {
  const int kind = gpt::gemm_split_count(d, side_by_side) > 1 ? GPT_K_GEMM_SPLITK : GPT_K_GEMM;
  LAUNCH(kind, site, 2.0 * d.M * d.N * d.K, 0, gpt::gemm(d, s, side_by_side));
  return GPT_OK;
}

#define GEMM(d, site)                             \
  do {                                            \
    int rc_ = run_gemm(m, s, (d), (site));        \
    if (rc_ != GPT_OK) return rc_;                \
  } while (0)
#define GEMM_SIDE(d, site, n)                     \
  do {                                            \
    int rc_ = run_gemm(m, s, (d), (site), (n));   \
    if (rc_ != GPT_OK) return rc_;                \
  } while (0)

// Visible (query, key) pairs of one (batch row, head).
double attn_pairs(int T, int left) {
  double n = 0;
  for (int i = 0; i < T; ++i) n += (left < 0 ? i : std::min(i, left)) + 1;
  return n;
}

// Parameter group g of the flat vector: 0 = embeddings, 1..L = layers,
// L + 1 = final LayerNorm and untied head.  Returns [begin, end).
void adam_group(const gpt_model* m, int g, int64_t* b, int64_t* e) {
  const int L = m->cfg.n_layer;
  auto start = [&](int k) -> int64_t {
    if (k == 0) return 0;
    if (k <= L) return m->pl.layer[k - 1].ln1w;
    if (k == L + 1) return m->pl.lnfw;
    return m->N;
  };
  *b = start(g);
  *e = start(g + 1);
}

// Make stream s wait for the side-stream AdamW of group g (all groups: g < 0).
int wait_adam(gpt_model* m, hipStream_t s, int g) {
  if (!m->adam_pending) return GPT_OK;
  const int idx = g < 0 ? (int)m->ev_adam.size() - 1 : g;
  hipError_t e = hipStreamWaitEvent(s, m->ev_adam[idx], 0);
  if (e != hipSuccess) return fail(GPT_E_HIP, std::string("hipStreamWaitEvent: ") + hipGetErrorString(e));
  if (g < 0) m->adam_pending = false;
  return GPT_OK;
}

int run_forward(gpt_model* m, const int32_t* idx, const int32_t* tgt, hipStream_t s) {
  const gpt_config& c = m->cfg;
  const int prec = m->prec();
  const int64_t M = m->M, C = m->C, F = m->F;
  const double act_b = m->bf16 ? 2.0 : 4.0;
  const double ln_fwd_bytes = M * C * (4.0 + act_b) + 8.0 * M;
  const double attn_flops = 4.0 * m->hd * m->B * m->H;
  auto act = [&](int64_t off) { return m->at<char>(off); };
  int rc = wait_adam(m, s, 0);
  if (rc != GPT_OK) return rc;
  const int32_t gen = ++m->gen;
  LAUNCH(GPT_K_EMBED, GPT_S_EMBED_FWD, 0, 12.0 * M * C,
         gpt::embed_fwd(prec, idx, m->P(m->pl.wte), m->P(m->pl.wpe), (int)M, m->T, (int)C,
                        c.vocab_size, m->X(0), m->at<int32_t>(m->ar.ids), m->id_flag(), gen, s));
  // The blocks run as FWD_CHAINS batch chains (for two: rows [0, M/2) on s,
  // the rest on fwdc[0]), issued layer by layer, so one chain's epilogues,
  // LayerNorms and attention overlap the other's products; every kernel is
  // row-independent, so the results are those of one chain.  Only for large
  // batches (small ones would change the products' plans); timed profiles
  // keep one stream.
  const int nch = (!m->prof_on && m->B % gpt_model::FWD_CHAINS == 0 &&
                   M / gpt_model::FWD_CHAINS >= 2048) ? gpt_model::FWD_CHAINS : 1;
  const int64_t Mh = M / nch;
  const int Bh = m->B / nch;
  const int64_t eb = m->bf16 ? 2 : 4;
  if (nch > 1) {
    hipError_t e = hipEventRecord(m->ev_ffork, s);
    for (int i = 0; i + 1 < nch && e == hipSuccess; ++i)
      e = hipStreamWaitEvent(m->fwdc[i], m->ev_ffork, 0);
    if (e != hipSuccess)
      return fail(GPT_E_HIP, std::string("forward fork: ") + hipGetErrorString(e));
  }
  auto block = [&](int l, int ch, hipStream_t s) -> int {
    const LayerOff& L = m->pl.layer[l];
    const int64_t r0 = ch * Mh;
    auto rows = [&](int64_t off, int64_t width) { return act(off) + r0 * width * eb; };
    int rc2 = wait_adam(m, s, 1 + l);
    if (rc2 != GPT_OK) return rc2;
    LAUNCH(GPT_K_LAYERNORM, GPT_S_LN_FWD, 0, ln_fwd_bytes / nch,
           gpt::layernorm_fwd(prec, m->X(2 * l) + r0 * C, m->P(L.ln1w), m->P(L.ln1b), (int)Mh,
                              (int)C, c.ln_eps, rows(m->ar.a1[l], C), m->mean(2 * l) + r0,
                              m->rstd(2 * l) + r0, s));
    gpt_gemm_desc d = linear_fwd(m, rows(m->ar.a1[l], C), C, L.qkvw, 3 * C, 3 * C);
    d.M = d.a_rows = (int)Mh;
    d.epilogue = GPT_EPI_STORE; d.bias = m->P(L.qkvb); d.out = rows(m->ar.qkv[l], 3 * C);
    d.ldo = 3 * C;
    GEMM_SIDE(d, GPT_S_QKV_FWD, nch);
    LAUNCH(GPT_K_ATTN_FWD, GPT_S_ATTN_FWD, attn_flops / nch * attn_pairs(m->T, c.window_left[l]), 0,
           gpt::attention_fwd(prec, Bh, m->T, (int)m->H, (int)m->hd, c.window_left[l],
                              rows(m->ar.qkv[l], 3 * C), rows(m->ar.att[l], C),
                              m->at<float>(m->ar.lse[l]) + (int64_t)ch * Bh * m->H * m->T, s));
    d = linear_fwd(m, rows(m->ar.att[l], C), C, L.projw, C, C);
    d.M = d.a_rows = (int)Mh;
    d.epilogue = GPT_EPI_RESIDUAL; d.bias = m->P(L.projb); d.resid = m->X(2 * l) + r0 * C;
    d.out = m->X(2 * l + 1) + r0 * C; d.ldo = C;
    GEMM_SIDE(d, GPT_S_PROJ_FWD, nch);
    LAUNCH(GPT_K_LAYERNORM, GPT_S_LN_FWD, 0, ln_fwd_bytes / nch,
           gpt::layernorm_fwd(prec, m->X(2 * l + 1) + r0 * C, m->P(L.ln2w), m->P(L.ln2b), (int)Mh,
                              (int)C, c.ln_eps, rows(m->ar.a2[l], C), m->mean(2 * l + 1) + r0,
                              m->rstd(2 * l + 1) + r0, s));
    d = linear_fwd(m, rows(m->ar.a2[l], C), C, L.fcw, F, F);
    d.M = d.a_rows = (int)Mh;
    // Kept for the backward: u itself when GELU is recomputed there, else
    // GELU'(u) (in the u buffer) next to GELU(u).
    d.epilogue = c.recompute_gelu ? GPT_EPI_GELU : GPT_EPI_GELU_PAIR;
    d.bias = m->P(L.fcb); d.out = rows(m->ar.u[l], F); d.ldo = F;
    d.aux = c.recompute_gelu ? nullptr : rows(m->ar.g[l], F); d.ldaux = F;
    GEMM_SIDE(d, GPT_S_FC_FWD, nch);
    if (c.recompute_gelu) {
      d = linear_fwd(m, rows(m->ar.u[l], F), F, L.fcpw, C, C);
      d.a_gelu = 1;
    } else {
      d = linear_fwd(m, rows(m->ar.g[l], F), F, L.fcpw, C, C);
    }
    d.M = d.a_rows = (int)Mh;
    d.epilogue = GPT_EPI_RESIDUAL; d.bias = m->P(L.fcpb); d.resid = m->X(2 * l + 1) + r0 * C;
    d.out = m->X(2 * l + 2) + r0 * C; d.ldo = C;
    GEMM_SIDE(d, GPT_S_FCPROJ_FWD, nch);
    return GPT_OK;
  };
  for (int l = 0; l < c.n_layer; ++l)
    for (int ch = 0; ch < nch; ++ch)
      if ((rc = block(l, ch, ch == 0 ? s : m->fwdc[ch - 1])) != GPT_OK) return rc;
  for (int i = 0; i + 1 < nch; ++i) {
    hipError_t e = hipEventRecord(m->ev_fjoin[i], m->fwdc[i]);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, m->ev_fjoin[i], 0);
    if (e != hipSuccess)
      return fail(GPT_E_HIP, std::string("forward join: ") + hipGetErrorString(e));
  }
  const int64_t nl = 2 * c.n_layer;
  if ((rc = wait_adam(m, s, -1)) != GPT_OK) return rc;  // the last group: all are done
  LAUNCH(GPT_K_LAYERNORM, GPT_S_LN_FWD, 0, ln_fwd_bytes,
         gpt::layernorm_fwd(prec, m->X(nl), m->P(m->pl.lnfw), m->P(m->pl.lnfb), (int)M, (int)C,
                            c.ln_eps, act(m->ar.xf), m->mean(nl), m->rstd(nl), s));
  gpt_gemm_desc d = linear_fwd(m, act(m->ar.xf), C, m->pl.lmw, m->Vq, m->Vp);
  d.epilogue = GPT_EPI_STORE; d.out = act(m->ar.logits); d.ldo = m->Vq;
  GEMM(d, GPT_S_LMHEAD_FWD);
  if (tgt) {
    LAUNCH(GPT_K_CROSS_ENTROPY, GPT_S_CROSS_ENTROPY, 0, 2.0 * M * m->Vq * act_b + 8.0 * M,
           gpt::cross_entropy(prec, act(m->ar.logits), (int)M, c.vocab_size, (int)m->Vq, tgt,
                              m->at<float>(m->ar.loss_rows), m->id_flag(), gen, s));
    LAUNCH(GPT_K_CROSS_ENTROPY, GPT_S_CROSS_ENTROPY, 0, 4.0 * M,
           gpt::mean_loss(m->at<float>(m->ar.loss_rows), (int)M, m->at<float>(m->ar.loss),
                          m->id_flag(), gen, s));
  }
  return GPT_OK;
}

int run_backward(gpt_model* m, int acc, hipStream_t s) {
  const gpt_config& c = m->cfg;
  const int prec = m->prec();
  const int64_t M = m->M, C = m->C, F = m->F;
  const double act_b = m->bf16 ? 2.0 : 4.0;
  const double ln_bwd_bytes = M * C * (2 * act_b + 12.0) + 8.0 * M;
  const double attn_flops = 8.0 * m->hd * m->B * m->H;
  auto act = [&](int64_t off) { return m->at<char>(off); };
  float* cs_part = m->at<float>(m->ar.cs_part);
  float* ln_part = m->at<float>(m->ar.ln_part);
  char* dC = act(m->ar.dC);
  char* dC2 = act(m->ar.dC2);
  int cur = 0;
  float* gres[2] = {m->at<float>(m->ar.gres[0]), m->at<float>(m->ar.gres[1])};

  // Weight and bias gradients only feed the optimizer: they run on the side
  // stream, overlapping the input-gradient chain on `s`.  While kernels are
  // being timed everything stays on `s`, so each kernel is timed alone.
  hipStream_t s2 = m->prof_on ? s : m->side;
  auto hip_ok = [&](hipError_t e, const char* what) -> int {
    return e == hipSuccess ? GPT_OK : fail(GPT_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  };
  auto fork = [&]() -> int {  // work enqueued on s so far is visible to s2
    if (s2 == s) return GPT_OK;
    int rc = hip_ok(hipEventRecord(m->ev_fork, s), "hipEventRecord");
    return rc != GPT_OK ? rc : hip_ok(hipStreamWaitEvent(s2, m->ev_fork, 0), "hipStreamWaitEvent");
  };
  // The gradients the weight-gradient branch reads live in rings: dF and dqkv
  // one slot per block (NGB deep), gact two per block.  The slots block l
  // writes were last read by the grouped launches of blocks l + 2 (the gact
  // its LayerNorm 1 writes), l + 3 (LayerNorm 2's) and l + NGB (dF, dqkv);
  // s2 runs those launches in order, so one wait per block, for block l + 2's
  // launch, frees them all (every event operation on s costs the chain a few
  // microseconds between its kernels).
  static_assert(NGB == 6, "the reuse distances above are those of rings of 6");
  auto group_done = [&](int l) -> int {  // s2 has read block l's buffers after this point
    if (s2 == s) return GPT_OK;
    return hip_ok(hipEventRecord(m->ev_buf[l % (3 * NGB)], s2), "hipEventRecord");
  };
  auto before_block = [&](int l) -> int {  // s may overwrite the slots block l writes
    if (s2 == s || l + 2 >= c.n_layer) return GPT_OK;
    return hip_ok(hipStreamWaitEvent(s, m->ev_buf[(l + 2) % (3 * NGB)], 0), "hipStreamWaitEvent");
  };
#define CHECK(x)                    \
  do {                              \
    int rc_ = (x);                  \
    if (rc_ != GPT_OK) return rc_;  \
  } while (0)
  auto gemm_on = [&](hipStream_t st, const gpt_gemm_desc& dd, int site) -> int {
    return run_gemm(m, st, dd, site);
  };
  auto gemm_group_on = [&](hipStream_t st, const gpt_gemm_desc* dd, float* const* db, int n,
                           int site, double* sq) -> int {
    double fl = 0;
    for (int i = 0; i < n; ++i) fl += 2.0 * dd[i].M * dd[i].N * dd[i].K;
    hipStream_t s = st;
    // The products and their fixed-order reduction are timed as separate sites.
    LAUNCH(GPT_K_GEMM_SPLITK, site, fl, 0, gpt::gemm_group(dd, n, s, db, 1));
    LAUNCH(GPT_K_GEMM_SPLITK, GPT_S_BLOCK_DW_REDUCE, 0, 0, gpt::gemm_group(dd, n, s, db, 2, sq));
    return GPT_OK;
  };
  // The gradient norm's partials: each block's grouped reduction writes its
  // rb per-block sums of squares at n_part + l * rb (every block has the same
  // shapes, so the same rb), the other ranges follow after the backward.
  m->norm_parts = false;
  double* n_part = m->at<double>(m->ar.n_part);
  bool fold = true;
  int rb = -1;
  auto bias_grad = [&](const char* x, int64_t n, int64_t off) -> int {
    if (off < 0) return GPT_OK;
    hipStream_t s = s2;
    LAUNCH(GPT_K_BIAS_GRAD, GPT_S_BIAS_GRAD, 0, M * n * act_b,
           gpt::colsum(prec, x, (int)M, (int)n, m->G(off), acc, cs_part, s));
    return GPT_OK;
  };

  // lm_head: dxf = dlogits . W ; dW (+)= dlogits^T . xf  (dlogits are in `logits`).
  const char* dlog = act(m->ar.logits);
  gpt_gemm_desc d = linear_dx(m, dlog, m->Vq, m->pl.lmw, C, m->Vq, m->Vp);
  d.epilogue = GPT_EPI_STORE; d.out = dC; d.ldo = C;
  d.workspace = m->at<void>(m->ar.gemm_ws);
  d.workspace_bytes = m->ar.gemm_ws_bytes;
  GEMM(d, GPT_S_LMHEAD_DX);
  CHECK(fork());
  d = linear_dw(m, dlog, m->Vq, m->Vq, act(m->ar.xf), C, m->pl.lmw, m->Vp, acc);
  CHECK(gemm_on(s2, d, GPT_S_LMHEAD_DW));
  if (s2 != s) CHECK(hip_ok(hipEventRecord(m->ev_lmdw, s2), "hipEventRecord"));
  const int64_t nl = 2 * c.n_layer;
  int gi = 0;  // gact[gi] holds the current LayerNorm input gradient (bf16); slots 0..NGB-1
  char* gact = act(m->ar.gact[gi]);
  LAUNCH(GPT_K_LAYERNORM, GPT_S_LN_BWD, 0, ln_bwd_bytes - 4.0 * M * C,
         gpt::layernorm_bwd(prec, dC, m->X(nl), m->mean(nl), m->rstd(nl), m->P(m->pl.lnfw), nullptr,
                            (int)M, (int)C, gres[cur], gact, m->G(m->pl.lnfw), m->G(m->pl.lnfb),
                            acc, ln_part, s));
  for (int l = c.n_layer - 1; l >= 0; --l) {
    const LayerOff& L = m->pl.layer[l];
    const int di = l % NGB;  // dF / dqkv ring slot: events NGB + di and 2 NGB + di
    char* dF = act(m->ar.dF[di]);
    char* dqkv = act(m->ar.dqkv[di]);
    // MLP out: x_out = x_mid + GELU(u) Wfcp^T + b
    CHECK(before_block(l));
    d = linear_dx(m, gact, C, L.fcpw, F, C, C);
    d.epilogue = c.recompute_gelu ? GPT_EPI_DGELU : GPT_EPI_MUL;
    d.aux = act(m->ar.u[l]); d.ldaux = F; d.out = dF; d.ldo = F;
    GEMM(d, GPT_S_FCPROJ_DX);
    // An event record on s costs the chain a few microseconds between its
    // kernels, so s2 is forked only where it launches next: here for the
    // float32 bias gradients and the recomputed-GELU weight gradient; in bf16
    // the block's products all wait for the fork after the attention.
    if (!m->bf16 || c.recompute_gelu) CHECK(fork());
    // The block's weight gradients share K (the tokens): they are collected
    // and issued as one grouped launch once dqkv exists, and the buffers they
    // read are released after it.  With GELU recompute the FC-projection
    // weight gradient applies GELU to its operand and runs alone.
    // In bf16 the bias gradients (column sums of each dY) come out of the same
    // launch, summed from the dY tiles it stages in LDS.
    gpt_gemm_desc dw[4];
    float* db[4];
    int ndw = 0;
    auto add_dw = [&](const gpt_gemm_desc& dd, const char* dy, int64_t n, int64_t b_off) -> int {
      dw[ndw] = dd;
      db[ndw] = (m->bf16 && b_off >= 0) ? m->G(b_off) : nullptr;
      ++ndw;
      return m->bf16 ? GPT_OK : bias_grad(dy, n, b_off);
    };
    if (c.recompute_gelu) {
      d = linear_dw(m, gact, C, C, act(m->ar.u[l]), F, L.fcpw, C, acc);
      d.b_gelu = 1;
      CHECK(gemm_on(s2, d, GPT_S_FCPROJ_DW));
      CHECK(bias_grad(gact, C, L.fcpb));
    } else {
      CHECK(add_dw(linear_dw(m, gact, C, C, act(m->ar.g[l]), F, L.fcpw, C, acc), gact, C, L.fcpb));
    }
    // MLP in: u = a2 Wfc^T + b
    CHECK(add_dw(linear_dw(m, dF, F, F, act(m->ar.a2[l]), C, L.fcw, F, acc), dF, F, L.fcb));
    d = linear_dx(m, dF, F, L.fcw, C, F, F);
    d.epilogue = GPT_EPI_STORE; d.out = dC; d.ldo = C;
    GEMM(d, GPT_S_FC_DX);
    gi = (gi + 1) % NGB;
    gact = act(m->ar.gact[gi]);
    LAUNCH(GPT_K_LAYERNORM, GPT_S_LN_BWD, 0, ln_bwd_bytes,
           gpt::layernorm_bwd(prec, dC, m->X(2 * l + 1), m->mean(2 * l + 1), m->rstd(2 * l + 1),
                              m->P(L.ln2w), gres[cur], (int)M, (int)C, gres[cur ^ 1], gact,
                              m->G(L.ln2w), m->G(L.ln2b), acc, ln_part, s));
    cur ^= 1;
    // attention out: x_mid = x_in + y Wproj^T + b
    if (!m->bf16) CHECK(fork());  // the float32 bias gradient of the projection
    CHECK(add_dw(linear_dw(m, gact, C, C, act(m->ar.att[l]), C, L.projw, C, acc), gact, C,
                 L.projb));
    d = linear_dx(m, gact, C, L.projw, C, C, C);
    d.epilogue = GPT_EPI_STORE; d.out = dC2; d.ldo = C;
    GEMM(d, GPT_S_PROJ_DX);
    LAUNCH(GPT_K_ATTN_BWD, GPT_S_ATTN_BWD, attn_flops * attn_pairs(m->T, c.window_left[l]), 0,
           gpt::attention_bwd(prec, m->B, m->T, (int)m->H, (int)m->hd, c.window_left[l],
                              act(m->ar.qkv[l]), act(m->ar.att[l]), m->at<float>(m->ar.lse[l]),
                              dC2, dqkv, m->at<float>(m->ar.dvec), s));
    // qkv = a1 Wqkv^T + b
    CHECK(fork());
    CHECK(add_dw(linear_dw(m, dqkv, 3 * C, 3 * C, act(m->ar.a1[l]), C, L.qkvw, 3 * C, acc), dqkv,
                 3 * C, L.qkvb));
    double* sq = nullptr;
    if (fold) {
      const int b = ndw == 4 ? gpt::gemm_group_reduce_blocks(dw, ndw, db) : 0;
      if (rb < 0) rb = b;
      fold = b > 0 && b == rb;
      if (fold) sq = n_part + (int64_t)l * rb;
    }
    CHECK(gemm_group_on(s2, dw, db, ndw, GPT_S_BLOCK_DW, sq));
    CHECK(group_done(l));
    d = linear_dx(m, dqkv, 3 * C, L.qkvw, C, 3 * C, 3 * C);
    d.epilogue = GPT_EPI_STORE; d.out = dC; d.ldo = C;
    GEMM(d, GPT_S_QKV_DX);
    gi = (gi + 1) % NGB;
    gact = act(m->ar.gact[gi]);
    LAUNCH(GPT_K_LAYERNORM, GPT_S_LN_BWD, 0, ln_bwd_bytes,
           gpt::layernorm_bwd(prec, dC, m->X(2 * l), m->mean(2 * l), m->rstd(2 * l), m->P(L.ln1w),
                              gres[cur], (int)M, (int)C, gres[cur ^ 1], gact, m->G(L.ln1w),
                              m->G(L.ln1b), acc, ln_part, s));
    cur ^= 1;
  }
  // x0 = wte[idx] + wpe[t]; with a tied head the lm_head gradient is already
  // in dwte: the embedding backward waits for that side-stream launch only,
  // and the rest of the side stream joins after it.
  if (s2 != s) CHECK(hip_ok(hipStreamWaitEvent(s, m->ev_lmdw, 0), "hipStreamWaitEvent"));
  gpt::EmbedBwdScratch scr{m->at<int32_t>(m->ar.e_counts),   m->at<int32_t>(m->ar.e_offsets),
                           m->at<int32_t>(m->ar.e_tile_sums), m->at<int32_t>(m->ar.e_rank),
                           m->at<int32_t>(m->ar.e_perm),
                           m->at<float>(m->ar.e_carry_first), m->at<float>(m->ar.e_carry_last),
                           m->at<int32_t>(m->ar.e_flags),    m->at<int32_t>(m->ar.e_last_tok)};
  const int wte_acc = (c.tied_lm_head || acc) ? 1 : 0;
  LAUNCH(GPT_K_EMBED, GPT_S_EMBED_BWD, 0, 4.0 * M * C + 4.0 * (m->Vp + c.block_size) * C,
         gpt::embed_bwd(m->at<int32_t>(m->ar.ids), gres[cur], (int)M, m->T, (int)C, (int)m->Vp,
                        c.block_size,
                        m->G(m->pl.wte), wte_acc, m->G(m->pl.wpe), acc, scr, s));
  // Every gradient is complete before anything after the backward runs.
  if (s2 != s) {
    CHECK(hip_ok(hipEventRecord(m->ev_join, s2), "hipEventRecord"));
    CHECK(hip_ok(hipStreamWaitEvent(s, m->ev_join, 0), "hipStreamWaitEvent"));
  }
  if (fold && rb > 0 && !m->norm_rng.empty()) {
    const int64_t off = (int64_t)c.n_layer * rb;
    LAUNCH(GPT_K_NORM, GPT_S_GRAD_NORM, 0, 0,
           gpt::sumsq_ranges(m->G(0), m->at<int64_t>(m->ar.n_rng), (int)(m->norm_rng.size() / 3),
                             m->norm_rng_blocks, n_part + off, s));
    m->norm_part_count = off + m->norm_rng_blocks;
    m->norm_parts = true;
  }
#undef CHECK
  return GPT_OK;
}

gpt::AdamScalars adam_scalars(const gpt_adamw_hp& hp) {
  gpt::AdamScalars sc;
  const double t = (double)hp.step_t;
  sc.omb1 = (float)(1.0 - hp.beta1);
  sc.omb2 = (float)(1.0 - hp.beta2);
  sc.decay = (float)(1.0 - hp.lr * hp.weight_decay);
  sc.step_size = (float)(hp.lr / (1.0 - std::pow(hp.beta1, t)));
  sc.sbc2 = (float)std::sqrt(1.0 - std::pow(hp.beta2, t));
  sc.eps = (float)hp.eps;
  sc.scale = (float)hp.grad_scale;
  return sc;
}

// The kinds of per-layer block matrix Muon updates: (offset in layer 0, rows, cols).
struct MuonKind { int64_t off0, off1; int rows, cols; };
std::vector<MuonKind> muon_kinds(const gpt_model* m) {
  const auto& L0 = m->pl.layer[0];
  const bool two = m->cfg.n_layer > 1;
  const auto* L1 = two ? &m->pl.layer[1] : nullptr;
  const int C = (int)m->C, F = (int)m->F;
  return {
      {L0.qkvw, two ? L1->qkvw : L0.qkvw, 3 * C, C},
      {L0.projw, two ? L1->projw : L0.projw, C, C},
      {L0.fcw, two ? L1->fcw : L0.fcw, F, C},
      {L0.fcpw, two ? L1->fcpw : L0.fcpw, C, F},
  };
}

int check_hp(const gpt_adamw_hp* hp) {
  if (!hp) return fail(GPT_E_INVALID, "hp is NULL");
  if (hp->step_t < 1) return fail(GPT_E_INVALID, "step_t must be >= 1");
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0 && hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return fail(GPT_E_INVALID, "betas must be in [0, 1)");
  if (!(hp->eps >= 0.0) || !std::isfinite(hp->lr) || !std::isfinite(hp->grad_scale))
    return fail(GPT_E_INVALID, "bad eps / lr / grad_scale");
  return GPT_OK;
}

}  // namespace

extern "C" {

const char* gpt_last_error(void) { return g_err.c_str(); }

double gpt_flops_per_token(const gpt_config* cfg, int32_t T) {
  if (!cfg || check_config(cfg, 1, T) != GPT_OK) return 0.0;
  return flops_per_token(*cfg, T);
}

int gpt_plan(const gpt_config* cfg, int32_t B, int32_t T, gpt_sizes* out) {
  int rc = check_config(cfg, B, T);
  if (rc != GPT_OK) return rc;
  if (!out) return fail(GPT_E_INVALID, "out is NULL");
  Arena a = plan_arena(*cfg, B, T);
  out->n_params = param_layout(*cfg).n;
  out->n_matmul_params = n_matmul(*cfg);
  out->flops_per_token = flops_per_token(*cfg, T);
  out->arena_bytes = a.total;
  out->state_bytes = a.state_end;
  out->activation_bytes = a.total - a.state_end;
  g_err.clear();
  return GPT_OK;
}

int gpt_init(const gpt_config* cfg, int32_t B, int32_t T, void* d_arena, int64_t arena_bytes,
             uint64_t seed, void* stream, gpt_model** out) {
  int rc = check_config(cfg, B, T);
  if (rc != GPT_OK) return rc;
  if (!out || !d_arena) return fail(GPT_E_INVALID, "NULL arena or out");
  if (((uintptr_t)d_arena) % ALIGN) return fail(GPT_E_INVALID, "arena must be 256-byte aligned");
  Arena a = plan_arena(*cfg, B, T);
  if (arena_bytes < a.total)
    return fail(GPT_E_INVALID, "arena too small: need " + std::to_string(a.total) + " bytes");
  gpt_model* m = new gpt_model();
  m->cfg = *cfg;
  m->B = B;
  m->T = T;
  m->M = (int64_t)B * T;
  m->C = cfg->n_embd;
  m->F = cfg->mlp_hidden;
  m->H = cfg->n_head;
  m->hd = m->C / m->H;
  m->Vp = cfg->padded_vocab;
  m->Vq = align_up(m->Vp, 64);
  m->bf16 = cfg->precision == GPT_BF16;
  m->pl = param_layout(*cfg);
  m->N = m->pl.n;
  m->ar = a;
  m->base = (char*)d_arena;
  m->state = 0;
  m->loss_valid = false;
  hipStream_t s = (hipStream_t)stream;
  hipError_t se = hipStreamCreateWithFlags(&m->side, hipStreamNonBlocking);
  if (se == hipSuccess) se = hipEventCreateWithFlags(&m->ev_fork, hipEventDisableTiming);
  if (se == hipSuccess) se = hipEventCreateWithFlags(&m->ev_join, hipEventDisableTiming);
  if (se == hipSuccess) se = hipEventCreateWithFlags(&m->ev_lmdw, hipEventDisableTiming);
  if (se == hipSuccess) se = hipEventCreateWithFlags(&m->ev_ffork, hipEventDisableTiming);
  for (int i = 0; i + 1 < gpt_model::FWD_CHAINS && se == hipSuccess; ++i) {
    se = hipStreamCreateWithFlags(&m->fwdc[i], hipStreamNonBlocking);
    if (se == hipSuccess) se = hipEventCreateWithFlags(&m->ev_fjoin[i], hipEventDisableTiming);
  }
  for (int i = 0; i < 3 * NGB && se == hipSuccess; ++i)
    se = hipEventCreateWithFlags(&m->ev_buf[i], hipEventDisableTiming);
  for (int i = 0; i < cfg->n_layer + 2 && se == hipSuccess; ++i) {
    hipEvent_t ev = nullptr;
    se = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (se == hipSuccess) m->ev_adam.push_back(ev);
  }
  if (se != hipSuccess) {
    gpt_destroy(m);
    return fail(GPT_E_HIP, std::string("side stream: ") + hipGetErrorString(se));
  }
  // Parameters, gradients, moments and the bf16 copy start at zero.  The
  // activation part is cleared too so padded logit columns read as zero.
  hipError_t e = hipMemsetAsync(d_arena, 0, (size_t)a.total, s);
  if (e != hipSuccess) {
    gpt_destroy(m);
    return fail(GPT_E_HIP, std::string("hipMemsetAsync: ") + hipGetErrorString(e));
  }
  // Seeded weights: matrices and embeddings N(0, 0.02) with the padded
  // vocabulary rows 0, LayerNorm gains 1 (shifts and biases stay 0).
  {
    const ParamLayout& pl = m->pl;
    const int64_t C = m->C, V = cfg->vocab_size;
    float* P0 = m->P(0);
    auto normal = [&](int64_t off, int64_t n, int64_t n_normal) {
      return gpt::init_normal(P0 + off, off, n, n_normal, 0.02, seed, s);
    };
    std::vector<std::pair<int64_t, int64_t>> gains = {{pl.lnfw, C}};
    e = normal(pl.wte, m->Vp * C, V * C);
    if (e == hipSuccess) e = normal(pl.wpe, (int64_t)cfg->block_size * C, (int64_t)cfg->block_size * C);
    for (int l = 0; l < cfg->n_layer && e == hipSuccess; ++l) {
      const LayerOff& L = pl.layer[l];
      gains.push_back({L.ln1w, C});
      gains.push_back({L.ln2w, C});
      for (auto w : {std::pair<int64_t, int64_t>{L.qkvw, 3 * C * C}, {L.projw, C * C},
                     {L.fcw, m->F * C}, {L.fcpw, C * m->F}})
        if (e == hipSuccess) e = normal(w.first, w.second, w.second);
    }
    if (e == hipSuccess && !cfg->tied_lm_head) e = normal(pl.lmw, m->Vp * C, V * C);
    for (auto gn : gains)
      if (e == hipSuccess) e = gpt::fill_value(P0 + gn.first, gn.second, 1.f, s);
    if (e == hipSuccess && m->bf16) e = gpt::to_bf16(P0, m->N, m->at<uint16_t>(a.shadow), s);
    if (e != hipSuccess) {
      gpt_destroy(m);
      return fail(GPT_E_HIP, std::string("parameter init: ") + hipGetErrorString(e));
    }
  }
  {
    std::vector<std::pair<int64_t, int64_t>> mr;
    for (int l = 0; l < cfg->n_layer; ++l)
      for (const MuonKind& k : muon_kinds(m)) {
        const int64_t b = k.off0 + l * (k.off1 - k.off0);
        mr.push_back({b, b + (int64_t)k.rows * k.cols});
      }
    std::sort(mr.begin(), mr.end());
    int64_t pos = 0;
    for (size_t i = 0; i <= mr.size(); ++i) {
      const int64_t end = i < mr.size() ? mr[i].first : m->N;
      if (end > pos) {
        m->adam_seg.insert(m->adam_seg.end(), {pos, end - pos, (int64_t)m->adam_seg_blocks});
        m->adam_seg_blocks += gpt::adamw_segment_blocks(end - pos);
      }
      if (i < mr.size()) pos = mr[i].second;
    }
    for (const auto& x : norm_ranges(m->cfg, m->pl)) {
      m->norm_rng.insert(m->norm_rng.end(), {x.first, x.second, (int64_t)m->norm_rng_blocks});
      m->norm_rng_blocks += gpt::sumsq_range_blocks(x.second);
    }
    // After the clear on the same stream; the host vectors live as long as the model.
    e = hipMemcpyAsync(m->at<int64_t>(a.adam_seg), m->adam_seg.data(), m->adam_seg.size() * 8,
                       hipMemcpyHostToDevice, s);
    if (e == hipSuccess && !m->norm_rng.empty())
      e = hipMemcpyAsync(m->at<int64_t>(a.n_rng), m->norm_rng.data(), m->norm_rng.size() * 8,
                         hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      gpt_destroy(m);
      return fail(GPT_E_HIP, std::string("hipMemcpy: ") + hipGetErrorString(e));
    }
  }
  *out = m;
  g_err.clear();
  return GPT_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- generation
struct gpt_gen {
  gpt_model* m;
  int B, Tmax, pos;
  char* base;
  int64_t kc, vc, x, a, qkv, att, u, gact, mean, rstd, logits, tok, ws, ws_bytes, posd, total;
  // The device copy of pos (posd) is what the kernels read; pos_dirty: the
  // host moved pos (reset) and the device copy is set before the next step.
  bool pos_dirty = false;
  // Decode steps after the token embedding replay one captured HIP graph
  // (captured on `cap` at the first step that needs it).
  bool use_graph = true;
  hipStream_t cap = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

namespace {

int64_t gen_layout(const gpt_model* m, int B, int Tmax, gpt_gen* g) {
  const int64_t act = m->bf16 ? 2 : 4, C = m->C, F = m->F, L = m->cfg.n_layer;
  int64_t o = 0;
  auto take = [&](int64_t bytes) { int64_t r = o; o = align_up(o + bytes, ALIGN); return r; };
  g->kc = take(L * B * m->H * Tmax * m->hd * act);
  g->vc = take(L * B * m->H * Tmax * m->hd * act);
  g->x = take(B * C * 4);
  g->a = take(B * C * act);
  g->qkv = take(B * 3 * C * act);
  g->att = take(B * C * act);
  g->u = take(B * F * act);
  g->gact = take(B * F * act);
  g->mean = take(B * 4);
  g->rstd = take(B * 4);
  g->logits = take(B * m->Vq * act);
  g->tok = take(B * 4);
  g->posd = take(16);
  // split-K partials of the fp32 decode products (at most 32 splits of B x max(3C, F) floats)
  g->ws_bytes = 32 * (int64_t)B * std::max(3 * C, F) * 4;
  g->ws = take(g->ws_bytes);
  g->total = o;
  return o;
}

int gen_check(const gpt_model* m, int B, int Tmax) {
  if (!m) return fail(GPT_E_INVALID, "NULL model");
  if (B < 1 || Tmax < 1 || Tmax > m->cfg.block_size)
    return fail(GPT_E_INVALID, "need B >= 1 and 1 <= Tmax <= block_size");
  if (!gpt::attn_decode_supported((int)m->hd))
    return fail(GPT_E_UNSUPPORTED, "head_dim must be 32, 64 or 128 for generation");
  return GPT_OK;
}

// out[B, N] = a[B, K] . W[N, K]^T with the given epilogue (rows of the decode step).
// One product of a decode step, optionally after a LayerNorm of the fp32 rows
// ln_x (ln_w set): bf16 runs the few-row MFMA kernel, which folds the
// LayerNorm in for K up to ROWS_LINEAR_MAX_LN_K; fp32 (and wider bf16 rows)
// run the LayerNorm kernel into a first.
hipError_t gen_linear(const gpt_gen* g, const void* a, int64_t K, int64_t w_off, int64_t N,
                      int64_t b_off, int epi, void* out, int64_t ldo, const float* resid,
                      void* aux, hipStream_t s, const float* ln_x = nullptr,
                      int64_t ln_w = -1, int64_t ln_b = -1) {
  const gpt_model* m = g->m;
  const bool fold_ln = ln_w >= 0 && m->bf16 && K <= gpt::ROWS_LINEAR_MAX_LN_K;
  if (ln_w >= 0 && !fold_ln) {
    const hipError_t e = gpt::layernorm_fwd(m->prec(), ln_x, m->P(ln_w), m->P(ln_b), g->B, (int)K,
                                            m->cfg.ln_eps, (void*)a, (float*)(g->base + g->mean),
                                            (float*)(g->base + g->rstd), s);
    if (e != hipSuccess) return e;
  }
  if (m->bf16) {
    gpt::RowsLinear p;
    if (fold_ln) {
      p.x = ln_x;
      p.ln_w = m->P(ln_w);
      p.ln_b = m->P(ln_b);
      p.eps = m->cfg.ln_eps;
    } else {
      p.a = a;
    }
    p.B = g->B; p.K = (int)K; p.N = (int)N;
    p.W = m->W(w_off);
    p.bias = b_off >= 0 ? m->P(b_off) : nullptr;
    p.epi = epi;
    p.out = out; p.ldo = ldo;
    p.resid = resid;
    p.aux = aux;
    p.tanh_form = m->cfg.gelu_tanh;
    return gpt::rows_linear(p, s);
  }
  gpt_gemm_desc d;
  std::memset(&d, 0, sizeof(d));
  d.precision = m->cfg.precision;
  d.gelu_tanh = m->cfg.gelu_tanh;
  d.M = g->B; d.N = (int)N; d.K = (int)K;
  d.A = a; d.lda = K; d.a_rows = g->B; d.a_kvalid = (int)K;
  d.B = m->W(w_off); d.ldb = K; d.b_rows = (int)N; d.b_kvalid = (int)K;
  d.epilogue = epi;
  d.bias = b_off >= 0 ? m->P(b_off) : nullptr;
  d.resid = resid;
  d.out = out; d.ldo = ldo;
  d.aux = aux; d.ldaux = aux ? ldo : 0;
  d.workspace = g->base + g->ws;
  d.workspace_bytes = g->ws_bytes;
  return gpt::gemm(d, s);
}

// Everything of a decode step after the token embedding (x already holds the
// embedded rows): the blocks, the final LayerNorm, the lm_head and the
// position advance.  Only kernel launches: it is captured into a graph.
int gen_body(gpt_gen* g, hipStream_t s) {
  gpt_model* m = g->m;
  const gpt_config& c = m->cfg;
  const int prec = m->prec();
  const int B = g->B;
  const int64_t C = m->C, F = m->F, act = m->bf16 ? 2 : 4;
  char* base = g->base;
  float* x = (float*)(base + g->x);
  void* a = base + g->a;
  float* mean = (float*)(base + g->mean);
  float* rstd = (float*)(base + g->rstd);
  const int64_t cache_layer = (int64_t)B * m->H * g->Tmax * m->hd * act;
  const int32_t* posd = (const int32_t*)(base + g->posd);
  for (int l = 0; l < c.n_layer; ++l) {
    const LayerOff& L = m->pl.layer[l];
    HIP_TRY(gen_linear(g, a, C, L.qkvw, 3 * C, L.qkvb, GPT_EPI_STORE, base + g->qkv, 3 * C,
                       nullptr, nullptr, s, x, L.ln1w, L.ln1b));
    HIP_TRY(gpt::attn_decode(prec, (int)m->hd, base + g->qkv, base + g->kc + l * cache_layer,
                             base + g->vc + l * cache_layer, posd, g->Tmax, B, (int)m->H,
                             c.window_left[l], base + g->att, s));
    HIP_TRY(gen_linear(g, base + g->att, C, L.projw, C, L.projb, GPT_EPI_RESIDUAL, x, C, x,
                       nullptr, s));
    HIP_TRY(gen_linear(g, a, C, L.fcw, F, L.fcb, GPT_EPI_GELU, base + g->u, F, nullptr,
                       base + g->gact, s, x, L.ln2w, L.ln2b));
    HIP_TRY(gen_linear(g, base + g->gact, F, L.fcpw, C, L.fcpb, GPT_EPI_RESIDUAL, x, C, x,
                       nullptr, s));
  }
  HIP_TRY(gpt::layernorm_fwd(prec, x, m->P(m->pl.lnfw), m->P(m->pl.lnfb), B, (int)C, c.ln_eps, a,
                             mean, rstd, s));
  HIP_TRY(gen_linear(g, a, C, m->pl.lmw, m->Vp, -1, GPT_EPI_STORE, base + g->logits, m->Vq,
                     nullptr, nullptr, s));
  HIP_TRY(gpt::gen_advance((int32_t*)(base + g->posd), s));
  return GPT_OK;
}

int gen_step(gpt_gen* g, const int32_t* d_tok, hipStream_t s) {
  gpt_model* m = g->m;
  if (g->pos >= g->Tmax) return fail(GPT_E_INVALID, "the cache is full (Tmax tokens)");
  int rc = wait_adam(m, s, -1);
  if (rc != GPT_OK) return rc;
  int32_t* posd = (int32_t*)(g->base + g->posd);
  if (g->pos_dirty) {
    HIP_TRY(gpt::gen_set_pos(posd, g->pos, s));
    g->pos_dirty = false;
  }
  HIP_TRY(gpt::gen_embed(d_tok, m->P(m->pl.wte), m->P(m->pl.wpe), posd, g->B, (int)m->C,
                         m->cfg.vocab_size, (float*)(g->base + g->x), s));
  if (!g->use_graph) {
    rc = gen_body(g, s);
    if (rc != GPT_OK) return rc;
  } else {
    if (!g->exec) {
      if (!g->cap) HIP_TRY(hipStreamCreateWithFlags(&g->cap, hipStreamNonBlocking));
      HIP_TRY(hipStreamBeginCapture(g->cap, hipStreamCaptureModeThreadLocal));
      rc = gen_body(g, g->cap);
      hipGraph_t graph = nullptr;
      const hipError_t ce = hipStreamEndCapture(g->cap, &graph);
      if (rc != GPT_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc;
      }
      if (ce != hipSuccess) return fail(GPT_E_HIP, std::string("capture: ") + hipGetErrorString(ce));
      g->graph = graph;
      HIP_TRY(hipGraphInstantiateWithFlags(&g->exec, g->graph, 0));
    }
    HIP_TRY(hipGraphLaunch(g->exec, s));
  }
  g->pos += 1;
  return GPT_OK;
}

}  // namespace

extern "C" {

int gpt_gen_plan(const gpt_model* m, int32_t B, int32_t Tmax, int64_t* bytes) {
  int rc = gen_check(m, B, Tmax);
  if (rc != GPT_OK) return rc;
  if (!bytes) return fail(GPT_E_INVALID, "NULL bytes");
  gpt_gen g;
  *bytes = gen_layout(m, B, Tmax, &g);
  return GPT_OK;
}

int gpt_gen_init(gpt_model* m, int32_t B, int32_t Tmax, void* d_arena, int64_t arena_bytes,
                 void* stream, gpt_gen** out) {
  int rc = gen_check(m, B, Tmax);
  if (rc != GPT_OK) return rc;
  if (!d_arena || !out) return fail(GPT_E_INVALID, "NULL arena or out");
  if (((uintptr_t)d_arena) % ALIGN) return fail(GPT_E_INVALID, "arena must be 256-byte aligned");
  gpt_gen* g = new gpt_gen();
  g->m = m;
  g->B = B;
  g->Tmax = Tmax;
  g->pos = 0;
  g->base = (char*)d_arena;
  if (arena_bytes < gen_layout(m, B, Tmax, g)) {
    delete g;
    return fail(GPT_E_INVALID, "generation arena too small");
  }
  hipError_t e = hipMemsetAsync(d_arena, 0, (size_t)g->total, (hipStream_t)stream);
  if (e != hipSuccess) {
    delete g;
    return fail(GPT_E_HIP, std::string("hipMemsetAsync: ") + hipGetErrorString(e));
  }
  *out = g;
  return GPT_OK;
}

int gpt_gen_set_graph(gpt_gen* g, int32_t enable) {
  if (!g || (enable != 0 && enable != 1)) return fail(GPT_E_INVALID, "NULL context or bad flag");
  g->use_graph = enable != 0;
  return GPT_OK;
}

int gpt_gen_reset(gpt_gen* g) {
  if (!g) return fail(GPT_E_INVALID, "NULL context");
  g->pos = 0;
  g->pos_dirty = true;
  return GPT_OK;
}

int gpt_gen_step(gpt_gen* g, const int32_t* d_tokens, void* stream) {
  if (!g || !d_tokens) return fail(GPT_E_INVALID, "NULL argument");
  return gen_step(g, d_tokens, (hipStream_t)stream);
}

int gpt_gen_logits(gpt_gen* g, void* h_dst, int64_t* ld, void* stream) {
  if (!g || !h_dst || !ld) return fail(GPT_E_INVALID, "NULL argument");
  const int64_t act = g->m->bf16 ? 2 : 4;
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(hipMemcpyAsync(h_dst, g->base + g->logits, (size_t)(g->B * g->m->Vq * act),
                         hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  *ld = g->m->Vq;
  return GPT_OK;
}

int gpt_gen_sample(gpt_gen* g, float temperature, int32_t top_k, const float* d_u,
                   int64_t u_stride, int32_t* d_tokens, void* stream) {
  if (!g || !d_tokens || (!d_u && temperature != 0.f)) return fail(GPT_E_INVALID, "NULL argument");
  if (!(temperature >= 0.f) || top_k < 0) return fail(GPT_E_INVALID, "bad temperature / top_k");
  if (g->pos == 0) return fail(GPT_E_STATE, "sample needs a step first");
  HIP_TRY(gpt::sample(g->m->prec(), g->base + g->logits, g->m->Vq, g->B, g->m->cfg.vocab_size,
                      temperature, top_k, d_u, u_stride, d_tokens, nullptr, 0, 0,
                      (hipStream_t)stream));
  return GPT_OK;
}

int gpt_generate(gpt_gen* g, const int32_t* d_prompt, int32_t T0, int32_t n_new,
                 float temperature, int32_t top_k, const float* d_uniforms, int32_t* d_out,
                 void* stream) {
  if (!g || !d_prompt || !d_out || (!d_uniforms && n_new > 0 && temperature != 0.f))
    return fail(GPT_E_INVALID, "NULL argument");
  if (T0 < 1 || n_new < 0 || T0 + n_new > g->Tmax)
    return fail(GPT_E_INVALID, "need T0 >= 1 and T0 + n_new <= Tmax");
  if (!(temperature >= 0.f) || top_k < 0) return fail(GPT_E_INVALID, "bad temperature / top_k");
  hipStream_t s = (hipStream_t)stream;
  const int Ltot = T0 + n_new;
  int32_t* tok = (int32_t*)(g->base + g->tok);
  g->pos = 0;
  g->pos_dirty = true;
  HIP_TRY(gpt::copy_prompt(d_prompt, T0, Ltot, g->B, d_out, s));
  for (int t = 0; t < T0; ++t) {
    HIP_TRY(gpt::gather_column(d_out, Ltot, t, g->B, tok, s));
    int rc = gen_step(g, tok, s);
    if (rc != GPT_OK) return rc;
  }
  for (int k = 0; k < n_new; ++k) {
    HIP_TRY(gpt::sample(g->m->prec(), g->base + g->logits, g->m->Vq, g->B,
                        g->m->cfg.vocab_size, temperature, top_k,
                        d_uniforms ? d_uniforms + k : nullptr, n_new, tok, d_out, Ltot, T0 + k, s));
    if (k + 1 < n_new) {
      int rc = gen_step(g, tok, s);
      if (rc != GPT_OK) return rc;
    }
  }
  return GPT_OK;
}

int gpt_gen_destroy(gpt_gen* g) {
  if (g) {
    if (g->exec) (void)hipGraphExecDestroy(g->exec);
    if (g->graph) (void)hipGraphDestroy(g->graph);
    if (g->cap) (void)hipStreamDestroy(g->cap);
  }
  delete g;
  return GPT_OK;
}

int gpt_destroy(gpt_model* m) {
  if (m) {
    for (hipEvent_t e : m->ev_pool) (void)hipEventDestroy(e);
    for (hipEvent_t e : {m->ev_fork, m->ev_join, m->ev_lmdw, m->ev_ffork})
      if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : m->ev_fjoin)
      if (e) (void)hipEventDestroy(e);
    for (hipStream_t f : m->fwdc)
      if (f) {
        (void)hipStreamSynchronize(f);
        (void)hipStreamDestroy(f);
      }
    for (hipEvent_t e : m->ev_buf)
      if (e) (void)hipEventDestroy(e);
    if (m->side) (void)hipStreamSynchronize(m->side);
    for (hipEvent_t e : m->ev_adam) (void)hipEventDestroy(e);
    if (m->side) (void)hipStreamDestroy(m->side);
  }
  delete m;
  return GPT_OK;
}

int gpt_forward(gpt_model* m, const int32_t* d_idx, const int32_t* d_tgt, void* stream) {
  if (!m || !d_idx) return fail(GPT_E_INVALID, "NULL model or idx");
  int rc = run_forward(m, d_idx, d_tgt, (hipStream_t)stream);
  if (rc != GPT_OK) return rc;
  if (d_tgt) {
    m->state = 1;
    m->loss_valid = true;
  } else {
    m->state = 0;
    m->loss_valid = false;
  }
  return GPT_OK;
}

int gpt_loss(gpt_model* m, void* stream, float* h_mean_loss) {
  if (!m || !h_mean_loss) return fail(GPT_E_INVALID, "NULL argument");
  if (!m->loss_valid) return fail(GPT_E_STATE, "no forward with targets since the last update");
  hipStream_t s = (hipStream_t)stream;
  int32_t flag = 0;
  HIP_TRY(hipMemcpyAsync(h_mean_loss, m->at<float>(m->ar.loss), 4, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipMemcpyAsync(&flag, m->id_flag(), 4, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  if (flag == m->gen)
    return fail(GPT_E_INVALID, "a token id or target of the last forward is outside [0, vocab_size)");
  return GPT_OK;
}

int gpt_loss_device_ptr(gpt_model* m, const float** d_loss) {
  if (!m || !d_loss) return fail(GPT_E_INVALID, "NULL argument");
  *d_loss = m->at<float>(m->ar.loss);
  return GPT_OK;
}

int gpt_backward(gpt_model* m, int32_t accumulate, void* stream) {
  if (!m) return fail(GPT_E_INVALID, "NULL model");
  if (m->state != 1) return fail(GPT_E_STATE, "backward needs a forward with targets first");
  if (accumulate != 0 && accumulate != 1) return fail(GPT_E_INVALID, "accumulate must be 0 or 1");
  int rc = run_backward(m, accumulate, (hipStream_t)stream);
  if (rc != GPT_OK) return rc;
  m->state = 2;
  return GPT_OK;
}

// The sum of squares of the gradient vector into norm2: from the backward's
// partials when it left them, else one fixed-order pass over the vector.
int grad_sumsq(gpt_model* m, hipStream_t s) {
  double* part = m->at<double>(m->ar.n_part);
  double* out = m->at<double>(m->ar.norm2);
  if (m->norm_parts) {
    LAUNCH(GPT_K_NORM, GPT_S_GRAD_NORM, 0, 8.0 * m->norm_part_count,
           gpt::sum_partials(part, (int)m->norm_part_count, out, s));
  } else {
    LAUNCH(GPT_K_NORM, GPT_S_GRAD_NORM, 0, 4.0 * m->N, gpt::sumsq(m->G(0), m->N, part, out, s));
  }
  return GPT_OK;
}

int gpt_grad_norm(gpt_model* m, void* stream, double* h_norm) {
  if (!m || !h_norm) return fail(GPT_E_INVALID, "NULL argument");
  if (m->state != 2) return fail(GPT_E_STATE, "grad_norm needs a backward first");
  hipStream_t s = (hipStream_t)stream;
  int rc = grad_sumsq(m, s);
  if (rc != GPT_OK) return rc;
  double n2 = 0.0;
  int32_t flag = 0;
  HIP_TRY(hipMemcpyAsync(&n2, m->at<double>(m->ar.norm2), 8, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipMemcpyAsync(&flag, m->id_flag(), 4, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  *h_norm = std::sqrt(n2);
  if (flag > m->upd_gen)
    return fail(GPT_E_INVALID, "a forward since the last update met a token id outside [0, vocab_size)");
  if (!std::isfinite(*h_norm)) return fail(GPT_E_NONFINITE, "gradient norm is not finite");
  return GPT_OK;
}

int gpt_adamw_step(gpt_model* m, const gpt_adamw_hp* hp, void* stream) {
  if (!m) return fail(GPT_E_INVALID, "NULL model");
  int rc = check_hp(hp);
  if (rc != GPT_OK) return rc;
  if (m->state != 2) return fail(GPT_E_STATE, "adamw_step needs a backward first");
  hipStream_t s = (hipStream_t)stream;
  float* pm = m->at<float>(m->ar.adam_m);
  float* pv = m->at<float>(m->ar.adam_v);
  uint16_t* sh = m->bf16 ? m->at<uint16_t>(m->ar.shadow) : nullptr;
  const gpt::AdamScalars sc = adam_scalars(*hp);
  if (m->prof_on) {  // timed alone, in one launch
    LAUNCH(GPT_K_ADAMW, GPT_S_ADAMW, 0, (m->bf16 ? 30.0 : 28.0) * m->N,
           gpt::adamw(m->N, m->P(0), pm, pv, m->G(0), sh, sc, s, nullptr, m->guard()));
  } else {
    // On the side stream, group by group; the next forward waits for each
    // group just before it uses those parameters.
    HIP_TRY(hipEventRecord(m->ev_fork, s));
    HIP_TRY(hipStreamWaitEvent(m->side, m->ev_fork, 0));
    for (int g = 0; g < (int)m->ev_adam.size(); ++g) {
      int64_t b, e;
      adam_group(m, g, &b, &e);
      HIP_TRY(gpt::adamw(e - b, m->P(b), pm + b, pv + b, m->G(b), sh ? sh + b : nullptr, sc,
                         m->side, nullptr, m->guard()));
      HIP_TRY(hipEventRecord(m->ev_adam[g], m->side));
    }
    m->adam_pending = true;
  }
  m->state = 0;
  m->loss_valid = false;
  m->upd_gen = m->gen;
  return GPT_OK;
}

int gpt_adamw_step_clipped(gpt_model* m, const gpt_adamw_hp* hp, int32_t n_micro, double max_norm,
                           double* h_norm_scale, void* stream) {
  if (!m) return fail(GPT_E_INVALID, "NULL model");
  int rc = check_hp(hp);
  if (rc != GPT_OK) return rc;
  if (n_micro < 1) return fail(GPT_E_INVALID, "n_micro must be >= 1");
  if (!(max_norm >= 0.0) || !std::isfinite(max_norm)) return fail(GPT_E_INVALID, "bad max_norm");
  if (m->state != 2) return fail(GPT_E_STATE, "adamw_step needs a backward first");
  hipStream_t s = (hipStream_t)stream;
  double* clip = m->at<double>(m->ar.clip);
  float* d_scale = (float*)(clip + 2);
  rc = grad_sumsq(m, s);
  if (rc != GPT_OK) return rc;
  HIP_TRY(gpt::clip_scale(m->at<double>(m->ar.norm2), n_micro, max_norm, clip, d_scale,
                          m->guard(), s));
  if (h_norm_scale)
    HIP_TRY(hipMemcpyAsync(h_norm_scale, clip, 16, hipMemcpyDeviceToHost, s));
  float* pm = m->at<float>(m->ar.adam_m);
  float* pv = m->at<float>(m->ar.adam_v);
  uint16_t* sh = m->bf16 ? m->at<uint16_t>(m->ar.shadow) : nullptr;
  const gpt::AdamScalars sc = adam_scalars(*hp);
  if (m->prof_on) {
    LAUNCH(GPT_K_ADAMW, GPT_S_ADAMW, 0, (m->bf16 ? 30.0 : 28.0) * m->N,
           gpt::adamw(m->N, m->P(0), pm, pv, m->G(0), sh, sc, s, d_scale));
  } else {
    HIP_TRY(hipEventRecord(m->ev_fork, s));
    HIP_TRY(hipStreamWaitEvent(m->side, m->ev_fork, 0));
    for (int g = 0; g < (int)m->ev_adam.size(); ++g) {
      int64_t b, e;
      adam_group(m, g, &b, &e);
      HIP_TRY(gpt::adamw(e - b, m->P(b), pm + b, pv + b, m->G(b), sh ? sh + b : nullptr, sc,
                         m->side, d_scale));
      HIP_TRY(hipEventRecord(m->ev_adam[g], m->side));
    }
    m->adam_pending = true;
  }
  m->state = 0;
  m->loss_valid = false;
  m->upd_gen = m->gen;
  return GPT_OK;
}

int gpt_loss_async(gpt_model* m, float* h_loss, void* stream) {
  if (!m || !h_loss) return fail(GPT_E_INVALID, "NULL argument");
  if (!m->loss_valid) return fail(GPT_E_STATE, "no forward with targets since the last update");
  HIP_TRY(hipMemcpyAsync(h_loss, m->at<float>(m->ar.loss), 4, hipMemcpyDeviceToHost,
                         (hipStream_t)stream));
  return GPT_OK;
}

int gpt_muon_step(gpt_model* m, const gpt_adamw_hp* adam, const gpt_muon_hp* muon,
                  void* stream) {
  if (!m) return fail(GPT_E_INVALID, "NULL model");
  int rc = check_hp(adam);
  if (rc != GPT_OK) return rc;
  if (!muon) return fail(GPT_E_INVALID, "muon hp is NULL");
  if (!(muon->momentum >= 0.0 && muon->momentum < 1.0 && muon->beta2 >= 0.0 &&
        muon->beta2 < 1.0) ||
      !(muon->eps >= 0.0) || !std::isfinite(muon->lr) || !std::isfinite(muon->weight_decay) ||
      muon->ns_steps < 0 || muon->ns_steps > 16)
    return fail(GPT_E_INVALID, "bad muon hyper-parameters");
  if (m->state != 2) return fail(GPT_E_STATE, "muon_step needs a backward first");
  hipStream_t s = (hipStream_t)stream;
  if ((rc = wait_adam(m, s, -1)) != GPT_OK) return rc;
  float* pm = m->at<float>(m->ar.adam_m);
  float* pv = m->at<float>(m->ar.adam_v);
  uint16_t* sh = m->bf16 ? m->at<uint16_t>(m->ar.shadow) : nullptr;
  const std::vector<MuonKind> kinds = muon_kinds(m);
  // AdamW on the runs of the flat vector between the Muon matrices, one launch.
  HIP_TRY(gpt::adamw_segments(m->at<int64_t>(m->ar.adam_seg), (int)(m->adam_seg.size() / 3),
                              m->adam_seg_blocks, m->P(0), pm, pv, m->G(0), sh,
                              adam_scalars(*adam), m->guard(), s));
  gpt::MuonScalars ms;
  ms.grad_scale = (float)adam->grad_scale;
  ms.mu = (float)muon->momentum;
  ms.omm = (float)(1.0 - muon->momentum);
  ms.omb2 = (float)(1.0 - muon->beta2);
  ms.eps = (float)muon->eps;
  ms.lr = (float)muon->lr;
  ms.lrwd = (float)(muon->lr * muon->weight_decay);
  ms.a = 3.4445f;
  ms.b = -4.7750f;
  ms.c = 2.0315f;
  ms.ns_steps = muon->ns_steps;
  for (const MuonKind& k : kinds) {
    gpt::MuonGroup g;
    g.g = m->G(k.off0);
    g.buf = pm + k.off0;
    g.v = pv + k.off0;
    g.p = m->P(k.off0);
    g.shadow = sh ? sh + k.off0 : nullptr;
    g.ls = (long)(k.off1 - k.off0);
    g.rows = k.rows;
    g.cols = k.cols;
    g.count = m->cfg.n_layer;
    HIP_TRY(gpt::muon_matrices(g, ms, m->prec(), m->at<void>(m->ar.muon_ws), m->guard(), s));
  }
  m->state = 0;
  m->loss_valid = false;
  m->upd_gen = m->gen;
  return GPT_OK;
}

static int buffer_region(gpt_model* m, int which, char** ptr, int64_t* bytes) {
  switch (which) {
    case GPT_BUF_PARAMS: *ptr = m->at<char>(m->ar.params); *bytes = m->N * 4; return GPT_OK;
    case GPT_BUF_GRADS: *ptr = m->at<char>(m->ar.grads); *bytes = m->N * 4; return GPT_OK;
    case GPT_BUF_ADAM_M: *ptr = m->at<char>(m->ar.adam_m); *bytes = m->N * 4; return GPT_OK;
    case GPT_BUF_ADAM_V: *ptr = m->at<char>(m->ar.adam_v); *bytes = m->N * 4; return GPT_OK;
    case GPT_BUF_LOSS_ROWS: *ptr = m->at<char>(m->ar.loss_rows); *bytes = m->M * 4; return GPT_OK;
  }
  return fail(GPT_E_INVALID, "unknown buffer id");
}

int gpt_get_buffer(gpt_model* m, int32_t which, void* dst, int32_t dst_on_device, void* stream) {
  if (!m || !dst) return fail(GPT_E_INVALID, "NULL argument");
  char* p;
  int64_t bytes;
  int rc = buffer_region(m, which, &p, &bytes);
  if (rc != GPT_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  if ((rc = wait_adam(m, s, -1)) != GPT_OK) return rc;
  HIP_TRY(hipMemcpyAsync(dst, p, (size_t)bytes,
                         dst_on_device ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToHost, s));
  if (!dst_on_device) HIP_TRY(hipStreamSynchronize(s));
  return GPT_OK;
}

int gpt_set_buffer(gpt_model* m, int32_t which, const void* src, int32_t src_on_device,
                   void* stream) {
  if (!m || !src) return fail(GPT_E_INVALID, "NULL argument");
  if (which == GPT_BUF_LOSS_ROWS) return fail(GPT_E_INVALID, "LOSS_ROWS is read-only");
  char* p;
  int64_t bytes;
  int rc = buffer_region(m, which, &p, &bytes);
  if (rc != GPT_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  if ((rc = wait_adam(m, s, -1)) != GPT_OK) return rc;
  HIP_TRY(hipMemcpyAsync(p, src, (size_t)bytes,
                         src_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, s));
  if (which == GPT_BUF_PARAMS && m->bf16)
    HIP_TRY(gpt::to_bf16(m->P(0), m->N, m->at<uint16_t>(m->ar.shadow), s));
  if (which == GPT_BUF_GRADS) {
    m->state = 2;  // caller-provided gradients may be stepped
    m->norm_parts = false;
  }
  if (!src_on_device) HIP_TRY(hipStreamSynchronize(s));
  return GPT_OK;
}

int gpt_profile_begin(gpt_model* m) {
  if (!m) return fail(GPT_E_INVALID, "NULL model");
  m->prof_on = true;
  m->recs.clear();
  m->ev_used = 0;
  return GPT_OK;
}

int gpt_profile_end(gpt_model* m, void* stream, gpt_kernel_stats* out, gpt_kernel_stats* sites) {
  if (!m || !out) return fail(GPT_E_INVALID, "NULL argument");
  m->prof_on = false;
  for (int k = 0; k < GPT_NUM_KERNEL_KINDS; ++k) out[k] = gpt_kernel_stats{0, 0.0, 0.0, 0.0};
  if (sites)
    for (int k = 0; k < GPT_NUM_SITES; ++k) sites[k] = gpt_kernel_stats{0, 0.0, 0.0, 0.0};
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
  for (const auto& r : m->recs) {
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b));
    for (gpt_kernel_stats* o : {&out[r.kind], sites ? &sites[r.site] : nullptr}) {
      if (!o) continue;
      o->launches += 1;
      o->ms += ms;
      o->flops += r.flops;
      o->bytes += r.bytes;
    }
  }
  m->recs.clear();
  m->ev_used = 0;
  return GPT_OK;
}

namespace {
int check_gemm_desc(const gpt_gemm_desc* d) {
  if (!d) return fail(GPT_E_INVALID, "NULL descriptor");
  if (d->precision != GPT_FP32 && d->precision != GPT_BF16)
    return fail(GPT_E_INVALID, "bad precision");
  if (d->epilogue < GPT_EPI_STORE || d->epilogue > GPT_EPI_AXPBY)
    return fail(GPT_E_INVALID, "bad epilogue");
  if (d->batch < 0) return fail(GPT_E_INVALID, "negative batch");
  if (d->batch > 1 && (d->bias || d->resid))
    return fail(GPT_E_INVALID, "batched products take no bias or resid");
  if (d->M < 0 || d->N < 0 || d->K < 0) return fail(GPT_E_INVALID, "negative size");
  if (!d->out && d->M > 0 && d->N > 0) return fail(GPT_E_INVALID, "NULL out");
  if (d->epilogue == GPT_EPI_RESIDUAL && !d->resid) return fail(GPT_E_INVALID, "NULL resid");
  if ((d->epilogue == GPT_EPI_DGELU || d->epilogue == GPT_EPI_GELU_PAIR ||
       d->epilogue == GPT_EPI_MUL || d->epilogue == GPT_EPI_AXPBY) && !d->aux)
    return fail(GPT_E_INVALID, "NULL aux");
  return GPT_OK;
}
}  // namespace

int gpt_op_gemm(const gpt_gemm_desc* d, void* stream) {
  int rc = check_gemm_desc(d);
  if (rc != GPT_OK) return rc;
  hipError_t e = gpt::gemm(*d, (hipStream_t)stream);
  if (e == hipErrorInvalidValue)
    return fail(GPT_E_INVALID, "gemm layout rule broken (K, lda, ldb must be multiples of 8)");
  if (e != hipSuccess) return fail(GPT_E_HIP, std::string("gemm: ") + hipGetErrorString(e));
  return GPT_OK;
}

int gpt_op_gemm_group(const gpt_gemm_desc* descs, float* const* bias_grads, int32_t n,
                      void* stream) {
  if (n < 1 || n > 4) return fail(GPT_E_INVALID, "group of 1..4 products");
  if (!descs) return fail(GPT_E_INVALID, "NULL descriptors");
  for (int i = 0; i < n; ++i) {
    int rc = check_gemm_desc(&descs[i]);
    if (rc != GPT_OK) return rc;
  }
  hipError_t e = gpt::gemm_group(descs, n, (hipStream_t)stream, bias_grads);
  if (e == hipErrorInvalidValue)
    return fail(GPT_E_INVALID, "gemm layout rule broken (K, lda, ldb multiples of 8; bias "
                               "gradients need a bf16 K-major A)");
  if (e != hipSuccess) return fail(GPT_E_HIP, std::string("gemm group: ") + hipGetErrorString(e));
  return GPT_OK;
}

int64_t gpt_op_gemm_group_workspace(const int32_t* M, const int32_t* N, int32_t n, int32_t K) {
  if (!M || !N || n < 1 || n > 4) return 0;
  return gpt::gemm_group_workspace_bytes(M, N, n, K);
}

int gpt_op_attention_fwd(int32_t precision, int32_t B, int32_t T, int32_t H, int32_t hd,
                         int32_t left, const void* qkv, void* out, float* lse, void* stream) {
  if (B < 0 || T < 0 || H < 0) return fail(GPT_E_INVALID, "negative size");
  if (!gpt::attention_supported(precision, hd)) return fail(GPT_E_UNSUPPORTED, "head_dim");
  HIP_TRY(gpt::attention_fwd(precision, B, T, H, hd, left, qkv, out, lse, (hipStream_t)stream));
  return GPT_OK;
}

int gpt_op_attention_bwd(int32_t precision, int32_t B, int32_t T, int32_t H, int32_t hd,
                         int32_t left, const void* qkv, const void* out, const float* lse,
                         const void* dout, void* dqkv, float* workspace, void* stream) {
  if (B < 0 || T < 0 || H < 0) return fail(GPT_E_INVALID, "negative size");
  if (!gpt::attention_supported(precision, hd)) return fail(GPT_E_UNSUPPORTED, "head_dim");
  HIP_TRY(gpt::attention_bwd(precision, B, T, H, hd, left, qkv, out, lse, dout, dqkv, workspace,
                             (hipStream_t)stream));
  return GPT_OK;
}

int gpt_op_attention_bwd_noalloc(int32_t precision, int32_t B, int32_t T, int32_t H, int32_t hd,
                                 int32_t left, const void* qkv, const void* out, const float* lse,
                                 const void* dout, void* dqkv, void* stream) {
  if (B < 0 || T < 0 || H < 0) return fail(GPT_E_INVALID, "negative size");
  if (!gpt::attention_supported(precision, hd)) return fail(GPT_E_UNSUPPORTED, "head_dim");
  const long need = 2L * B * H * T;
  if (need > gpt::ATTN_SCRATCH_FLOATS)
    return fail(GPT_E_INVALID, "B*H*T = " + std::to_string((long)B * H * T) +
                                   " exceeds the static scratch (at most " +
                                   std::to_string(gpt::ATTN_SCRATCH_FLOATS / 2) + " rows)");
  float* ws = nullptr;
  HIP_TRY(gpt::attention_scratch(need, &ws));
  HIP_TRY(gpt::attention_bwd(precision, B, T, H, hd, left, qkv, out, lse, dout, dqkv, ws,
                             (hipStream_t)stream));
  return GPT_OK;
}

int gpt_op_adamw(int64_t n, float* p, float* m, float* v, const float* g, uint16_t* shadow,
                 const gpt_adamw_hp* hp, void* stream) {
  int rc = check_hp(hp);
  if (rc != GPT_OK) return rc;
  if (n < 0) return fail(GPT_E_INVALID, "negative n");
  if (n > 0 && (!p || !m || !v || !g)) return fail(GPT_E_INVALID, "NULL array");
  if ((((uintptr_t)p) | ((uintptr_t)m) | ((uintptr_t)v) | ((uintptr_t)g)) % 16 ||
      ((uintptr_t)shadow) % 8)
    return fail(GPT_E_INVALID, "arrays must be 16-byte aligned (shadow 8-byte)");
  HIP_TRY(gpt::adamw(n, p, m, v, g, shadow, adam_scalars(*hp), (hipStream_t)stream));
  return GPT_OK;
}

}  // extern "C"
