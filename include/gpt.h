/*
 * gpt.h — C ABI of the MI355X (gfx950) decoder-only GPT training step.
 *
 * One training step of a GPT of the nanoGPT / llm.c kind: learned token and
 * position embeddings, pre-LayerNorm blocks of causal (optionally sliding-
 * window) multi-head self-attention and a GELU MLP, final LayerNorm, a tied or
 * untied lm_head and the mean cross-entropy loss; then the exact gradient, the
 * global gradient norm and an AdamW update of float32 master weights.
 *
 * Sources (web pages, by title and section):
 *   - nanoGPT README, "quick start" / "reproducing GPT-2" / "todos": the model
 *     (6-layer, 6-head, 384-channel character model; GPT-2 124M; absolute
 *     learned position embeddings, other schemes listed under "todos");
 *   - Panthalia "Create a Plugin", "Components of the Example Plugin": the
 *     GPTConfig fields and the flattened-tensor representation of the model
 *     that forward/backward/update act on;
 *   - NiNo README, "usage": the call order model(data) -> cross_entropy ->
 *     backward -> step -> zero_grad;
 *   - nanochat "Architektur im Überblick", "FLOPs-Berechnung im Detail" (FLOP
 *     formula, per-layer (left, right) windows) and "AdamW Fused Step" (the
 *     update order and host-side hyper-parameters that change without a
 *     rebuild);
 *   - llm.c summary "Reimplementando el modelo GPT-2 ...", "Proceso de
 *     entrenamiento" (gradient clipping) and "Ejecución del entrenamiento"
 *     (the -r recompute option).
 *
 * Conventions (all entry points):
 *   - Return a gpt_status; no exception crosses the ABI.  On error the
 *     thread-local message from gpt_last_error() says what failed.
 *   - "device" pointers are HIP device addresses on the current device;
 *     "host" pointers are ordinary CPU memory.
 *   - Every launch is enqueued on the given hipStream_t (passed as void*;
 *     NULL is the null stream).  Only gpt_loss, gpt_grad_norm and the
 *     host-side variants of gpt_get_buffer / gpt_set_buffer synchronise.
 *   - Ownership: the caller allocates the single device arena whose size
 *     gpt_plan reports, and keeps it alive until gpt_destroy.  The library
 *     borrows it and owns only the opaque host handle.
 *   - Token ids and targets must lie in [0, vocab_size).  The kernels never
 *     index out of bounds with others: they read id 0 in their place, the
 *     forward is flagged, its mean loss reads NaN, gpt_loss / gpt_grad_norm
 *     return GPT_E_INVALID, and the next optimizer step (gpt_adamw_step,
 *     gpt_adamw_step_clipped, gpt_muon_step) leaves parameters and moments
 *     unchanged.  A later update after clean forwards proceeds normally.
 */
#ifndef GPT_MI355X_H
#define GPT_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GPT_MAX_LAYERS 128

typedef enum gpt_status {
  GPT_OK = 0,
  GPT_E_INVALID = 1,     /* bad argument or configuration                 */
  GPT_E_STATE = 2,       /* call out of order (e.g. backward before forward) */
  GPT_E_HIP = 3,         /* a HIP runtime call failed                      */
  GPT_E_NONFINITE = 4,   /* gradient norm is NaN or Inf                    */
  GPT_E_UNSUPPORTED = 5  /* valid but not implemented (e.g. head_dim 48)   */
} gpt_status;

typedef enum gpt_precision { GPT_FP32 = 0, GPT_BF16 = 1 } gpt_precision;

/* Model hyper-parameters (the GPTConfig of the Panthalia plugin example).
 * Linear weights are [out, in] row-major.  n_embd % 64 == 0, mlp_hidden % 64
 * == 0, n_embd % n_head == 0; the bf16 path needs head_dim in {32, 64, 128}. */
typedef struct gpt_config {
  int32_t vocab_size;     /* real vocabulary: softmax over [0, vocab_size)          */
  int32_t padded_vocab;   /* rows of wte / lm_head (>= vocab_size); pad rows are 0  */
  int32_t block_size;     /* rows of wpe; T <= block_size                           */
  int32_t n_layer, n_head, n_embd, mlp_hidden;
  int32_t bias;           /* 1: LayerNorm shifts and Linear biases exist            */
  int32_t tied_lm_head;   /* 1: lm_head is wte                                      */
  int32_t gelu_tanh;      /* 1: tanh-approximated GELU, 0: exact erf GELU           */
  int32_t precision;      /* gpt_precision                                          */
  int32_t recompute_gelu; /* 1: GELU(u) is recomputed instead of stored             */
  float ln_eps;           /* LayerNorm epsilon (1e-5)                               */
  int32_t window_left[GPT_MAX_LAYERS]; /* per layer: key j visible to query i iff
                                          i - left <= j <= i; < 0 = full causal  */
} gpt_config;

/* Sizes for one (config, B, T).  All byte counts are for the device arena. */
typedef struct gpt_sizes {
  int64_t n_params;         /* float32 entries of the flat parameter vector           */
  int64_t n_matmul_params;  /* parameters that enter a matmul (the FLOP formula's N)  */
  double flops_per_token;   /* 6 * n_matmul_params + sum_l 12 * h * q * T_eff          */
  int64_t arena_bytes;      /* one device allocation, 256-byte aligned base           */
  int64_t state_bytes;      /* params + grads + m + v (+ bf16 shadow) part of it     */
  int64_t activation_bytes; /* saved activations + backward scratch                   */
} gpt_sizes;

/* Which flat float32 buffer gpt_get_buffer / gpt_set_buffer address.  All
 * are n_params entries in the flat order: wte, wpe, then per layer ln1.w,
 * [ln1.b], qkv.w, [qkv.b], proj.w, [proj.b], ln2.w, [ln2.b], fc.w, [fc.b],
 * fcproj.w, [fcproj.b], then lnf.w, [lnf.b], then lm_head.w when untied
 * (bracketed entries only when bias = 1).  GPT_BUF_LOSS_ROWS is B*T floats
 * (per-token loss of the last forward with targets). */
typedef enum gpt_buffer {
  GPT_BUF_PARAMS = 0, GPT_BUF_GRADS = 1, GPT_BUF_ADAM_M = 2, GPT_BUF_ADAM_V = 3,
  GPT_BUF_LOSS_ROWS = 4
} gpt_buffer;

/* AdamW hyper-parameters, host doubles.  Each per-step scalar (1-beta1,
 * 1-beta2, 1-lr*wd, lr/(1-beta1^t), sqrt(1-beta2^t), eps, grad_scale) is
 * computed in double and rounded once to float.  Per element, in float32
 * with no fused multiply-add:
 *   g *= grad_scale; p *= 1-lr*wd; m += (1-beta1)*(g-m); v += (1-beta2)*(g*g-v);
 *   p -= step_size * (m / (sqrt(v)/sqrt(1-beta2^t) + eps))
 * and the bf16 weight copy (bf16 mode) is refreshed from p. */
typedef struct gpt_adamw_hp {
  double lr, beta1, beta2, eps, weight_decay;
  double grad_scale;  /* clipping factor; 1.0 = no clipping                      */
  int64_t step_t;     /* 1-based step count for the bias corrections            */
} gpt_adamw_hp;

/* Muon hyper-parameters (nanochat "Optimierungsstrategien Muon und AdamW").
 * For each per-layer Linear weight W [rows, cols] with gradient G:
 *   g = G * grad_scale; buf += (1-momentum)(g - buf); u = g + momentum (buf - g)
 *   X = act(u) / (||X||_F * 1.01 + 1e-6); then ns_steps times, with
 *   (a, b, c) = (3.4445, -4.7750, 2.0315):
 *     rows > cols: A = X^T X, B = b A + c A A, X = a X + X B
 *     otherwise:   A = X X^T, B = b A + c A A, X = a X + B X
 *   s_i = mean of X^2 over the shorter dimension (i along the longer one);
 *   v_i += (1-beta2)(s_i - v_i); Y = X / (sqrt(v_i) + eps), rescaled to ||X||_F;
 *   W -= lr Y + lr weight_decay W [Y W >= 0]   (cautious decay).
 * The momentum buffer is the matrix's ADAM_M slot and v the first
 * max(rows, cols) entries of its ADAM_V slot.  bf16 mode: X, A and B are bf16
 * (the page's iteration runs in bf16); fp32 mode: float. */
typedef struct gpt_muon_hp {
  double lr, momentum, beta2, weight_decay, eps;
  int32_t ns_steps;   /* 0..16 */
} gpt_muon_hp;

typedef struct gpt_model gpt_model;

/* Host only.  Validates cfg and (B, T) and fills *out.  INVALID on a bad
 * config (n_embd % n_head != 0, T > block_size, padded_vocab < vocab_size,
 * ...), UNSUPPORTED for shapes the kernels do not cover. */
int gpt_plan(const gpt_config* cfg, int32_t B, int32_t T, gpt_sizes* out);

/* Nanochat FLOP formula per token at sequence length T (host only; 0 on a
 * bad config). */
double gpt_flops_per_token(const gpt_config* cfg, int32_t T);

/* Bind a model to a caller-owned device arena of at least arena_bytes
 * (gpt_plan), 256-byte aligned, and initialise it on `stream` for training
 * from scratch (nanoGPT README, "quick start"; the pages fix no initial scale,
 * so the usual GPT-2 scale 0.02 is taken): every matrix and embedding entry at
 * flat index i is
 * (float)(0.02 * z(i)), z(i) a standard normal drawn from `seed` by
 * Philox4x32-10 (Salmon et al., SC 2011; block i / 4, counter (i/4 lo, i/4 hi,
 * 0, 0), key (seed lo, seed hi)) and the Box-Muller transform in double (words
 * 0, 1 -> entries 4j, 4j+1 as r cos, r sin; words 2, 3 -> 4j+2, 4j+3); the
 * padded vocabulary rows (>= vocab_size) of wte / lm_head are 0, LayerNorm
 * gains 1, LayerNorm shifts and Linear biases 0.  Gradients and both moments
 * start at 0.  The same seed gives the same bits.  Other weights can be
 * loaded with gpt_set_buffer(GPT_BUF_PARAMS).  Synchronises `stream`.
 * INVALID for a bad config, a NULL or misaligned arena or one too small;
 * HIP on a failed launch. */
int gpt_init(const gpt_config* cfg, int32_t B, int32_t T, void* d_arena, int64_t arena_bytes,
             uint64_t seed, void* stream, gpt_model** out);

/* Forward pass (NiNo README "usage": output = model(data); nanoGPT README
 * "quick start": the GPT of model.py) on device token ids d_idx [B*T]
 * (int32, row-major [B][T], caller-owned and read during the enqueued work
 * only).  With d_tgt [B*T] (int32, the next-token targets: Panthalia "Create
 * a Plugin", input-target pairs) the per-token cross-entropy (NiNo README,
 * "usage": the mean cross-entropy of the output against the target) and its
 * gradient w.r.t. the logits are computed too (required before gpt_backward);
 * with d_tgt == NULL only the logits.  Ids outside [0, vocab_size): see the
 * conventions above.
 * Enqueue only.  INVALID on NULL model / d_idx. */
int gpt_forward(gpt_model* m, const int32_t* d_idx, const int32_t* d_tgt, void* stream);

/* Mean loss of the last forward with targets (NiNo README "usage": the mean
 * cross-entropy; llm.c summary "Proceso de entrenamiento": the loss printed
 * per iteration), summed in double in a fixed order.  Synchronises `stream`.
 * STATE if there is no forward with targets since the last update; INVALID
 * (with *h_mean_loss = NaN) if that forward met an id outside [0, vocab_size). */
int gpt_loss(gpt_model* m, void* stream, float* h_mean_loss);

/* Device address of that mean loss (one float), valid after gpt_forward
 * with targets has been enqueued; for callers that avoid a sync. */
int gpt_loss_device_ptr(gpt_model* m, const float** d_loss);

/* The mean loss of the last forward with targets, copied to host memory
 * h_loss asynchronously on `stream` (valid once the stream has passed this
 * point; page-locked memory keeps the call asynchronous). */
int gpt_loss_async(gpt_model* m, float* h_loss, void* stream);

/* Backward pass of the last forward with targets (NiNo README "usage":
 * loss.backward(); Panthalia "Create a Plugin": gradient computation on the
 * flattened representation): the exact gradient of the mean loss w.r.t. every
 * parameter, into the flat gradient buffer.  accumulate = 0 overwrites it,
 * 1 adds to it (gradient accumulation over micro-batches, as in the
 * Panthalia plugin example).  Enqueue only.  STATE without a preceding forward with
 * targets; INVALID for accumulate not in {0, 1}. */
int gpt_backward(gpt_model* m, int32_t accumulate, void* stream);

/* Global L2 norm of the gradient buffer (llm.c summary "Proceso de
 * entrenamiento": the gradient norm that clipping acts on), float32 squares
 * summed per workgroup, workgroups summed in double in a fixed order (in bf16
 * the blocks' weight and bias gradients are squared by the backward's own
 * fixed-order reductions as it stores them; gradients written with
 * gpt_set_buffer are summed in one pass).  Synchronises.
 * Returns GPT_E_NONFINITE (with *h_norm set) if the norm is NaN or Inf;
 * STATE without a backward; INVALID (with *h_norm set) if a forward since
 * the last update met an id outside [0, vocab_size). */
int gpt_grad_norm(gpt_model* m, void* stream, double* h_norm);

/* One AdamW update of all parameters (see gpt_adamw_hp).  Enqueue only. */
int gpt_adamw_step(gpt_model* m, const gpt_adamw_hp* hp, void* stream);

/* Gradient-norm clipping and the AdamW update with no host round trip
 * (llm.c / nanoGPT "train_gpt2": clip the global gradient norm at
 * max_norm before the optimizer step).  Enqueue only.  On the device: norm =
 * sqrt(sum g^2) / n_micro (the norm of the mean of n_micro accumulated
 * micro-batch gradients), c = max_norm / norm if max_norm > 0 and
 * norm > max_norm, else 1, grad_scale = c / n_micro; hp->grad_scale is
 * ignored.  The arithmetic is gpt_grad_norm followed by that host rule in
 * double, so the update is bit-identical to gpt_adamw_step with the
 * host-computed grad_scale.  A non-finite norm leaves parameters, moments and
 * the bf16 copy unchanged.  h_norm_scale: NULL or host memory for {norm,
 * grad_scale} (NaN scale: non-finite norm), copied asynchronously on
 * `stream`; page-locked memory keeps the call asynchronous. */
int gpt_adamw_step_clipped(gpt_model* m, const gpt_adamw_hp* hp, int32_t n_micro, double max_norm,
                           double* h_norm_scale, void* stream);

/* The hybrid optimizer step (after gpt_backward, in place of gpt_adamw_step):
 * Muon (hp `muon`, above) on every per-layer Linear weight, AdamW (hp
 * `adam`, including its grad_scale and step_t) on every other tensor
 * (embeddings, LayerNorm and bias vectors, the untied lm_head).  Runs on
 * `stream`; uses a Muon region of the arena.  Errors as gpt_adamw_step. */
int gpt_muon_step(gpt_model* m, const gpt_adamw_hp* adam, const gpt_muon_hp* muon, void* stream);

/* Copy a flat buffer out of (get) or into (set) the model.  `dst`/`src` is
 * host memory when *_on_device == 0 (the call then synchronises), device
 * memory otherwise.  Setting PARAMS also refreshes the bf16 weight copy.
 * LOSS_ROWS is read-only. */
int gpt_get_buffer(gpt_model* m, int32_t which, void* dst, int32_t dst_on_device, void* stream);
int gpt_set_buffer(gpt_model* m, int32_t which, const void* src, int32_t src_on_device,
                   void* stream);

/* ------------------------------------------------------------------------
 * Kernel timing.  Between gpt_profile_begin and gpt_profile_end every kernel
 * launch of the step is bracketed by HIP events on its stream, and
 * gpt_profile_end (which synchronises) sums, per kernel kind, the launches,
 * the elapsed milliseconds, and the algorithmic FLOPs and HBM bytes of those
 * launches (FLOPs: 2*M*N*K per matrix product, 4*hd (forward) or 8*hd
 * (backward) per visible (query, key) pair of attention; bytes: the minimal
 * reads + writes of the memory-bound kernels).  Calls outside a profile
 * window launch no events.
 * ---------------------------------------------------------------------- */
typedef enum gpt_kernel_kind {
  GPT_K_GEMM = 0,          /* MFMA / fp32 matrix product, one kernel            */
  GPT_K_GEMM_SPLITK = 1,   /* split-K matrix product + its fixed-order reduce    */
  GPT_K_ATTN_FWD = 2,
  GPT_K_ATTN_BWD = 3,      /* D = rowsum(dO*O), dK/dV kernel, dQ kernel          */
  GPT_K_LAYERNORM = 4,     /* forward and backward (incl. gain/shift reduce)     */
  GPT_K_CROSS_ENTROPY = 5, /* fused softmax-CE + dlogits, and the loss mean      */
  GPT_K_EMBED = 6,         /* embedding forward and backward                     */
  GPT_K_BIAS_GRAD = 7,     /* column sums for Linear bias gradients              */
  GPT_K_NORM = 8,          /* gradient sum of squares                            */
  GPT_K_ADAMW = 9,
  GPT_NUM_KERNEL_KINDS = 10
} gpt_kernel_kind;

typedef struct gpt_kernel_stats {
  int64_t launches;
  double ms, flops, bytes;
} gpt_kernel_stats;

/* Call sites of the step (one per distinct launch in the layer loop).  Each
 * matrix-product site maps to exactly one kernel specialisation. */
typedef enum gpt_site {
  GPT_S_EMBED_FWD = 0, GPT_S_LN_FWD, GPT_S_QKV_FWD, GPT_S_ATTN_FWD, GPT_S_PROJ_FWD,
  GPT_S_FC_FWD, GPT_S_FCPROJ_FWD, GPT_S_LMHEAD_FWD, GPT_S_CROSS_ENTROPY, GPT_S_LMHEAD_DX,
  GPT_S_LMHEAD_DW, GPT_S_LN_BWD, GPT_S_FCPROJ_DX, GPT_S_FCPROJ_DW, GPT_S_FC_DX, GPT_S_FC_DW,
  GPT_S_PROJ_DX, GPT_S_PROJ_DW, GPT_S_ATTN_BWD, GPT_S_QKV_DX, GPT_S_QKV_DW, GPT_S_BIAS_GRAD,
  GPT_S_EMBED_BWD, GPT_S_GRAD_NORM, GPT_S_ADAMW,
  GPT_S_BLOCK_DW,  /* a block's four weight gradients as one grouped launch (split partials) */
  GPT_S_BLOCK_DW_REDUCE,  /* ... and the fixed-order reduction of its partials and bias sums */
  GPT_NUM_SITES
} gpt_site;

int gpt_profile_begin(gpt_model* m);
/* out: GPT_NUM_KERNEL_KINDS entries; sites (may be NULL): GPT_NUM_SITES entries. */
int gpt_profile_end(gpt_model* m, void* stream, gpt_kernel_stats* out, gpt_kernel_stats* sites);

/* Release the host handle (the arena stays the caller's). */
int gpt_destroy(gpt_model* m);

/* ---- Generation with a key/value cache (nanoGPT README, "sampling /
 * inference"; llm.c summary, "Sampling").  A generation context reads the
 * weights of a model (bf16 copy in bf16 mode, float32 in fp32 mode; they must
 * not change while it is used) and owns a caller-provided device arena with
 * the caches [n_layer][B][n_head][Tmax][head_dim] (act type) of B sequences
 * and the activations of one decode step.  Every call is enqueued on
 * `stream`; none synchronises unless stated. */
typedef struct gpt_gen gpt_gen;

/* Device bytes of a generation arena for B sequences of up to Tmax tokens
 * (1 <= Tmax <= block_size).  GPT_E_UNSUPPORTED if head_dim is not 32/64/128. */
int gpt_gen_plan(const gpt_model* m, int32_t B, int32_t Tmax, int64_t* bytes);
/* Create a context on `d_arena` (256-byte aligned, >= gpt_gen_plan bytes,
 * caller-owned).  The host handle is freed by gpt_gen_destroy. */
int gpt_gen_init(gpt_model* m, int32_t B, int32_t Tmax, void* d_arena, int64_t arena_bytes,
                 void* stream, gpt_gen** out);
/* Forget the cached tokens (next gpt_gen_step is position 0). */
int gpt_gen_reset(gpt_gen* g);
/* Decode steps replay one captured HIP graph (enable = 1, the default) or
 * launch their kernels one by one (0); the results are the same bits.  The
 * token embedding of a step is launched on its own (its token buffer is the
 * caller's per step); the rest of the step (every block, the final LayerNorm,
 * the lm_head) is captured at the first step that needs it, on a stream of
 * the context, and reads the position from device memory, so the one graph
 * serves every position (nanoGPT README "sampling / inference": sampling
 * from a trained model; the llm.c summary notes the code is not optimised
 * for inference).  INVALID for a NULL context or a flag other than 0 / 1. */
int gpt_gen_set_graph(gpt_gen* g, int32_t enable);
/* Append one token per sequence (d_tokens: device int32 [B], ids < vocab)
 * at the current position: its keys / values join the cache and the logits
 * of the next token are computed.  GPT_E_INVALID once Tmax tokens are cached. */
int gpt_gen_step(gpt_gen* g, const int32_t* d_tokens, void* stream);
/* Copy the last step's logits [B][ld] to host memory (synchronous): element
 * type is the act type (bf16 bits in bf16 mode, float in fp32 mode); *ld
 * receives the row pitch in elements (>= vocab_size; entries >= vocab_size
 * are padding). */
int gpt_gen_logits(gpt_gen* g, void* h_dst, int64_t* ld, void* stream);
/* Draw one token per sequence from the last step's logits: temperature 0 =
 * argmax (lowest index on ties); otherwise softmax of logits/temperature over
 * the top_k largest (0 = all; ties at the threshold kept), token = the
 * smallest i whose cumulative probability exceeds d_u[b*u_stride] (device
 * float in [0, 1)).  Writes d_tokens[b] (device int32 [B]). */
int gpt_gen_sample(gpt_gen* g, float temperature, int32_t top_k, const float* d_u,
                   int64_t u_stride, int32_t* d_tokens, void* stream);
/* Reset, feed the prompt d_prompt [B][T0] one position at a time, then draw
 * n_new tokens (draw s of row b uses d_uniforms[b*n_new + s]); d_out [B][T0 +
 * n_new] receives the prompt and the continuation.  T0 >= 1, T0 + n_new <= Tmax. */
int gpt_generate(gpt_gen* g, const int32_t* d_prompt, int32_t T0, int32_t n_new,
                 float temperature, int32_t top_k, const float* d_uniforms, int32_t* d_out,
                 void* stream);
int gpt_gen_destroy(gpt_gen* g);

/* Message of the last failed call on this thread ("" if none). */
const char* gpt_last_error(void);

/* ------------------------------------------------------------------------
 * Single-operation entry points (the kernels of the step, exposed for
 * unit parity).  Precision: GPT_FP32 = float operands, GPT_BF16 = bf16
 * operands with float accumulation.
 * ---------------------------------------------------------------------- */

/* Epilogues of C = op(A) . op(B)^T (op(A) is M x K, op(B) is N x K). */
typedef enum gpt_epilogue {
  GPT_EPI_STORE = 0,      /* out(act)  = acc [+ bias]                               */
  GPT_EPI_RESIDUAL = 1,   /* out(f32)  = resid + acc [+ bias]                       */
  GPT_EPI_GELU = 2,       /* out(act)  = u = acc [+ bias]; aux(act) = GELU(u) if aux */
  GPT_EPI_DGELU = 3,      /* out(act)  = acc * GELU'(aux[m, n])                     */
  GPT_EPI_F32 = 4,        /* out(f32)  = acc                                        */
  GPT_EPI_F32_ACCUM = 5,  /* out(f32) += acc                                        */
  GPT_EPI_GELU_PAIR = 6,  /* u = acc [+ bias] rounded to act; out(act) = GELU'(u),
                             aux(act) = GELU(u) (aux required)                       */
  GPT_EPI_MUL = 7,        /* out(act)  = acc * aux[m, n] (aux required)             */
  GPT_EPI_AXPBY = 8       /* out(act)  = alpha * acc + beta * aux[m, n] (aux required) */
} gpt_epilogue;

/* One matrix product, nanoGPT Linear convention (y = x W^T).  Operand X (A or
 * B) is "row-major over K" when x_trans == 0: element (r, k) at X[r*ldx + k];
 * "K-major" when x_trans == 1: element (r, k) at X[k*ldx + r].  Elements with
 * r >= x_rows or k >= x_kvalid read as zero (for x_trans == 1 the check on r
 * is per group of 8, so X must stay finite and allocated up to a multiple of
 * 8 past x_rows).  Every leading dimension % 8 == 0, and K % 8 == 0 unless both
 * operands are K-major.
 * a_gelu / b_gelu = 1 apply GELU to that operand as it is read.  Split-K
 * partial sums (deterministic, fixed order) use `workspace` when K is long;
 * workspace_bytes == 0 disables splitting. */
typedef struct gpt_gemm_desc {
  int32_t precision, M, N, K;
  const void* A; int64_t lda; int32_t a_trans, a_rows, a_kvalid, a_gelu;
  const void* B; int64_t ldb; int32_t b_trans, b_rows, b_kvalid, b_gelu;
  int32_t epilogue, gelu_tanh;
  const float* bias;    /* [N] or NULL                                  */
  const float* resid;   /* [M, ldo] float, RESIDUAL only                 */
  void* out; int64_t ldo;
  void* aux; int64_t ldaux;  /* GELU output / DGELU input, act type     */
  void* workspace; int64_t workspace_bytes;
  float alpha, beta;    /* AXPBY scalars (ignored by the other epilogues)        */
  /* batch > 1: `batch` independent products of the same shape; matrix z reads
   * A + z*stride_a, B + z*stride_b, aux + z*stride_aux and writes
   * out + z*stride_out (byte strides).  Batched products are never split
   * over K and take no bias or resid.  batch 0 or 1: one product. */
  int32_t batch;
  int64_t stride_a, stride_b, stride_out, stride_aux;
} gpt_gemm_desc;

int gpt_op_gemm(const gpt_gemm_desc* d, void* stream);

/* n (1..4) products sharing K in one launch, as a transformer block's weight
 * gradients dW (+)= dY^T X are (the backward of the step's Linear layers,
 * nanoGPT "model.py" CausalSelfAttention / MLP; K = the batch's tokens).  Each
 * descriptor is validated as in gpt_op_gemm.  Grouped when every product is
 * bf16 with both operands K-major (a_trans = b_trans = 1), epilogue F32 or
 * F32_ACCUM (the same for all), no bias / resid / GELU operand / batch, and
 * descs[0].workspace holds the split partials (gpt_op_gemm_group_workspace);
 * the 256-tiles of all products are split over K together and each product's
 * partial sums are reduced in fixed split order, so results are reproducible
 * (not bitwise equal to gpt_op_gemm, whose split count differs).  Otherwise
 * the products run one by one through gpt_op_gemm.  bias_grads: NULL, or n
 * device pointers (entries may be NULL): bias_grads[i][m] (+)= sum over k of
 * A_i(m, k), the Linear bias gradient when A_i = dY, stored or added as
 * product i's epilogue; taken from the operand tiles the grouped kernel has
 * in LDS (requires a bf16 K-major A_i, else GPT_E_INVALID).  descs and
 * bias_grads are host memory, read during the call only. */
int gpt_op_gemm_group(const gpt_gemm_desc* descs, float* const* bias_grads, int32_t n,
                      void* stream);
/* Workspace bytes the grouped launch of products [M_i, N_i] with reduction
 * length K needs, bias-gradient partials included (0 if n is out of range). */
int64_t gpt_op_gemm_group_workspace(const int32_t* M, const int32_t* N, int32_t n, int32_t K);

/* Causal (windowed) attention over a packed qkv [B*T, 3*H*hd] (q | k | v,
 * head h at columns h*hd of each third).  out [B*T, H*hd] (act type), lse
 * [B, H, T] float = log-sum-exp of the scaled scores per query.
 * left < 0: full causal, else key j visible to query i iff i-left <= j <= i. */
int gpt_op_attention_fwd(int32_t precision, int32_t B, int32_t T, int32_t H, int32_t hd,
                         int32_t left, const void* qkv, void* out, float* lse, void* stream);

/* Gradient of gpt_op_attention_fwd: dout [B*T, H*hd] -> dqkv [B*T, 3*H*hd].
 * `workspace` holds 2*B*H*T floats (device, caller-owned; overwritten). */
int gpt_op_attention_bwd(int32_t precision, int32_t B, int32_t T, int32_t H, int32_t hd,
                         int32_t left, const void* qkv, const void* out, const float* lse,
                         const void* dout, void* dqkv, float* workspace, void* stream);

/* gpt_op_attention_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same result, bit for bit, with no
 * workspace argument.  D and the log2-unit log-sum-exp live in a static
 * device array of 2^21 floats (8 MiB) per GPU, held until the process ends,
 * so B*H*T <= 1,048,576; larger sizes return GPT_E_INVALID before any launch.
 * The call allocates nothing (no hipMalloc / hipFree / allocating library
 * call).  Every call on one GPU shares that array: calls that overlap on one
 * GPU (concurrent streams, threads) race; calls ordered on one stream are
 * safe.  Nothing in the array needs to start at zero. */
int gpt_op_attention_bwd_noalloc(int32_t precision, int32_t B, int32_t T, int32_t H, int32_t hd,
                                 int32_t left, const void* qkv, const void* out, const float* lse,
                                 const void* dout, void* dqkv, void* stream);

/* The AdamW update on raw device float arrays of n entries; `shadow`
 * (bf16, n entries) is written when non-NULL. */
int gpt_op_adamw(int64_t n, float* p, float* m, float* v, const float* g, uint16_t* shadow,
                 const gpt_adamw_hp* hp, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPT_MI355X_H */
