"""Plain NumPy oracle of one decoder-only GPT training step — TEST INFRASTRUCTURE.

Only tests, the smoke check and the benchmark's CPU-baseline leg use this file.
It is deliberately slow and literal: dense T x T attention per (batch, head),
the exact softmax, a hand-derived reverse pass written out op by op, and an
AdamW update done one correctly rounded float32 operation at a time.

What it follows (page titles and sections of the source pages):
  * nanoGPT README ("quick start", "reproducing GPT-2", "todos"): a GPT with
    learned token and position embeddings, pre-LayerNorm transformer blocks of
    causal multi-head self-attention and an MLP, tied lm_head, `bias` switch;
  * Panthalia "Create a Plugin" (the `GPTConfig` example and "Components"):
    block_size / vocab_size / n_layer / n_head / n_embd / bias, the flattened
    parameter representation, input/target pairs;
  * NiNo README ("usage"): the loss is the mean cross-entropy of the logits
    against the targets;
  * nanochat "Architektur im Überblick", "FLOPs-Berechnung im Detail": FLOPs
    per token = 6 * (params - excluded) + sum over layers 12*h*q*effective_seq,
    with a (left, right) window per layer; "AdamW Fused Step": decay, lerp of
    the first moment, bias correction, update p -= step_size * m / denom;
  * llm.c summary ("Proceso de entrenamiento"): gradient clipping.

Readings where the pages are silent (each also listed in the design notes):
  LayerNorm eps 1e-5 with biased variance; "GELU" is the exact erf form and
  "GELU(tanh)" the tanh approximation; the window admits key j for query i iff
  i - left <= j <= i; padded vocabulary columns are excluded from the softmax;
  the second moment uses the same lerp as the first, denom = sqrt(v)/sqrt(1 -
  beta2^t) + eps; clipping scale = min(1, max_norm / ||g||) without epsilon.

Every function takes plain arrays; nothing here is shared with the device path.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy.special import erf

__all__ = [
    "FlopCounter", "layout", "n_params", "n_matmul_params", "flops_per_token",
    "unflatten", "flatten", "forward", "backward", "loss_and_grads", "grad_norm",
    "clip_scale", "adamw_scalars", "adamw_update", "bf16_round", "bf16_bits",
    "layernorm_fwd", "layernorm_bwd", "gelu", "gelu_grad", "attention_fwd",
    "attention_bwd", "cross_entropy_fwd_bwd", "visible", "step", "logits",
    "loss_rows", "cosine_lr", "train_steps", "NS_COEFFS", "muon_matrices",
    "orthogonalize", "muon_momentum", "muon_second_moment", "cautious_update",
    "muon_matrix_update", "MuonHP", "muon_hybrid_step", "sample_token", "next_token_logits",
    "generate", "philox4x32_10", "philox_normals", "init_params",
]


# --------------------------------------------------------------------------
# bookkeeping
# --------------------------------------------------------------------------
class FlopCounter:
    """Counts 2*m*n*k for every matrix product the oracle performs."""

    def __init__(self):
        self.flops = 0

    def mm(self, a, b):
        out = np.matmul(a, b)
        m, k = a.shape[-2], a.shape[-1]
        n = b.shape[-1]
        batch = int(np.prod(out.shape[:-2])) if out.ndim > 2 else 1
        self.flops += 2 * batch * m * n * k
        return out


def _mm(ctr, a, b):
    return ctr.mm(a, b) if ctr is not None else np.matmul(a, b)


def layout(cfg):
    """(name, shape) of every parameter tensor, in the flat order of the
    Panthalia page's flat form of the model's parameters (one contiguous vector)."""
    C, F, Vp, Tb = cfg["n_embd"], cfg["mlp_hidden"], cfg["padded_vocab"], cfg["block_size"]
    bias = bool(cfg["bias"])
    out = [("wte", (Vp, C)), ("wpe", (Tb, C))]
    for l in range(cfg["n_layer"]):
        p = f"h{l}."
        out += [(p + "ln1.w", (C,))] + ([(p + "ln1.b", (C,))] if bias else [])
        out += [(p + "qkv.w", (3 * C, C))] + ([(p + "qkv.b", (3 * C,))] if bias else [])
        out += [(p + "proj.w", (C, C))] + ([(p + "proj.b", (C,))] if bias else [])
        out += [(p + "ln2.w", (C,))] + ([(p + "ln2.b", (C,))] if bias else [])
        out += [(p + "fc.w", (F, C))] + ([(p + "fc.b", (F,))] if bias else [])
        out += [(p + "fcproj.w", (C, F))] + ([(p + "fcproj.b", (C,))] if bias else [])
    out += [("lnf.w", (C,))] + ([("lnf.b", (C,))] if bias else [])
    if not cfg["tied"]:
        out.append(("lm_head.w", (Vp, C)))
    return out


def n_params(cfg) -> int:
    return sum(int(np.prod(s)) for _, s in layout(cfg))


def n_matmul_params(cfg) -> int:
    """Parameters that enter a matrix product: the per-layer Linear weights and
    the lm_head matrix (the token embedding itself when tied).  Embedding
    look-ups and 0-D/1-D tensors are the "excluded" parameters of the nanochat
    FLOP formula."""
    total = 0
    for name, shape in layout(cfg):
        if len(shape) == 2 and name not in ("wte", "wpe", "lm_head.w"):
            total += int(np.prod(shape))
    total += cfg["padded_vocab"] * cfg["n_embd"]  # the lm_head matmul
    return total


def flops_per_token(cfg, T: int) -> int:
    """nanochat "FLOPs-Berechnung im Detail": 6*(N - N_excluded) + sum_l 12*h*q*T_eff,
    T_eff = T for a full layer, min(window, T) for a windowed one."""
    h = cfg["n_head"]
    q = cfg["n_embd"] // h
    attn = 0
    for w in cfg["window_left"]:
        eff = T if w < 0 else min(w, T)
        attn += 12 * h * q * eff
    return 6 * n_matmul_params(cfg) + attn


def unflatten(cfg, flat, dtype=np.float64):
    flat = np.asarray(flat)
    P, off = {}, 0
    for name, shape in layout(cfg):
        n = int(np.prod(shape))
        P[name] = flat[off:off + n].astype(dtype).reshape(shape)
        off += n
    if off != flat.size:
        raise ValueError(f"flat vector has {flat.size} entries, layout needs {off}")
    return P


def flatten(cfg, tensors, dtype=np.float64):
    return np.concatenate([np.asarray(tensors[name], dtype=dtype).reshape(-1)
                           for name, _ in layout(cfg)])


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------
def layernorm_fwd(x, w, b, eps):
    """LayerNorm over the last axis: (x - mean) / sqrt(biased var + eps) * w + b."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * rstd
    y = xhat * w
    if b is not None:
        y = y + b
    return y, xhat, rstd


def layernorm_bwd(dy, xhat, rstd, w):
    """Exact gradient of layernorm_fwd.  Returns dx, dw, db."""
    dxhat = dy * w
    C = dy.shape[-1]
    dx = rstd * (dxhat - dxhat.sum(-1, keepdims=True) / C
                 - xhat * (dxhat * xhat).sum(-1, keepdims=True) / C)
    dw = (dy * xhat).reshape(-1, C).sum(0)
    db = dy.reshape(-1, C).sum(0)
    return dx, dw, db


_S2PI = math.sqrt(2.0 / math.pi)
_K = 0.044715


def gelu(u, tanh_form: bool):
    """GELU.  Exact: u * Phi(u).  tanh form: 0.5 u (1 + tanh(sqrt(2/pi)(u + 0.044715 u^3)))."""
    if tanh_form:
        return 0.5 * u * (1.0 + np.tanh(_S2PI * (u + _K * u ** 3)))
    return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))


def gelu_grad(u, tanh_form: bool):
    if tanh_form:
        t = np.tanh(_S2PI * (u + _K * u ** 3))
        return 0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * _S2PI * (1.0 + 3.0 * _K * u * u)
    phi = np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)
    return 0.5 * (1.0 + erf(u / math.sqrt(2.0))) + u * phi


def visible(T: int, left: int):
    """mask[i, j] = key j is visible to query i: j <= i and i - j <= left (left < 0: no limit).
    This is the (left, right=0) window of nanochat's "Sliding Window" listing."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    m = j <= i
    if left >= 0:
        m &= (i - j) <= left
    return m


def attention_fwd(q, k, v, left: int, ctr=None):
    """Causal (optionally windowed) softmax attention for one sequence.
    q, k, v: [H, T, hd].  Returns y [H, T, hd] and the probabilities P [H, T, T]."""
    H, T, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    S = _mm(ctr, q, np.swapaxes(k, -1, -2)) * scale
    mask = visible(T, left)
    S = np.where(mask, S, -np.inf)
    mx = S.max(axis=-1, keepdims=True)
    E = np.exp(S - mx)
    P = E / E.sum(axis=-1, keepdims=True)
    y = _mm(ctr, P, v)
    return y, P


def attention_bwd(dy, q, k, v, P, ctr=None):
    """Gradient of attention_fwd w.r.t. q, k, v (masked entries have P = 0)."""
    hd = q.shape[-1]
    scale = 1.0 / math.sqrt(hd)
    dP = _mm(ctr, dy, np.swapaxes(v, -1, -2))
    dv = _mm(ctr, np.swapaxes(P, -1, -2), dy)
    dS = P * (dP - (dP * P).sum(-1, keepdims=True))
    dq = _mm(ctr, dS, k) * scale
    dk = _mm(ctr, np.swapaxes(dS, -1, -2), q) * scale
    return dq, dk, dv


def cross_entropy_fwd_bwd(z, tgt, V: int, n_total: int):
    """Per-row loss logsumexp_{v<V} z - z[tgt] and d(mean loss)/dz; columns >= V
    are padding and take part in neither."""
    zr = z[:, :V]
    mx = zr.max(axis=1, keepdims=True)
    e = np.exp(zr - mx)
    s = e.sum(axis=1, keepdims=True)
    lse = (mx + np.log(s))[:, 0]
    rows = np.arange(z.shape[0])
    loss_r = lse - z[rows, tgt]
    dz = np.zeros_like(z)
    dz[:, :V] = e / s
    dz[rows, tgt] -= 1.0
    dz /= n_total
    return loss_r, dz


# --------------------------------------------------------------------------
# the model
# --------------------------------------------------------------------------
def _lm_weight(cfg, P):
    return P["wte"] if cfg["tied"] else P["lm_head.w"]


def forward(cfg, P, idx, ctr=None):
    """Forward pass up to the logits.  P: dict of arrays (unflatten).  Returns (z, cache)."""
    B, T = idx.shape
    C, H = cfg["n_embd"], cfg["n_head"]
    hd = C // H
    eps = cfg.get("ln_eps", 1e-5)
    bias = bool(cfg["bias"])
    tanh_form = bool(cfg["gelu_tanh"])
    BT = B * T
    x = (P["wte"][idx] + P["wpe"][:T][None, :, :]).reshape(BT, C)
    cache = {"layers": []}
    for l in range(cfg["n_layer"]):
        p = f"h{l}."
        Lc = {"x_in": x}
        a1, Lc["xhat1"], Lc["rstd1"] = layernorm_fwd(x, P[p + "ln1.w"], P.get(p + "ln1.b"), eps)
        qkv = _mm(ctr, a1, P[p + "qkv.w"].T)
        if bias:
            qkv = qkv + P[p + "qkv.b"]
        q, k, v = (qkv[:, i * C:(i + 1) * C].reshape(B, T, H, hd).transpose(0, 2, 1, 3)
                   for i in range(3))
        y = np.empty((B, H, T, hd), dtype=x.dtype)
        probs = []
        for b in range(B):
            y[b], Pb = attention_fwd(q[b], k[b], v[b], cfg["window_left"][l], ctr)
            probs.append(Pb)
        y2 = y.transpose(0, 2, 1, 3).reshape(BT, C)
        x = x + _mm(ctr, y2, P[p + "proj.w"].T)
        if bias:
            x = x + P[p + "proj.b"]
        Lc.update(a1=a1, q=q, k=k, v=v, probs=probs, y2=y2, x_mid=x)
        a2, Lc["xhat2"], Lc["rstd2"] = layernorm_fwd(x, P[p + "ln2.w"], P.get(p + "ln2.b"), eps)
        u = _mm(ctr, a2, P[p + "fc.w"].T)
        if bias:
            u = u + P[p + "fc.b"]
        g = gelu(u, tanh_form)
        x = x + _mm(ctr, g, P[p + "fcproj.w"].T)
        if bias:
            x = x + P[p + "fcproj.b"]
        Lc.update(a2=a2, u=u, g=g)
        cache["layers"].append(Lc)
    xf, cache["xhatf"], cache["rstdf"] = layernorm_fwd(x, P["lnf.w"], P.get("lnf.b"), eps)
    z = _mm(ctr, xf, _lm_weight(cfg, P).T)
    cache.update(xf=xf, idx=idx, B=B, T=T)
    return z, cache


def backward(cfg, P, cache, dz, ctr=None):
    """Reverse pass from dL/dlogits to a dict of parameter gradients."""
    B, T = cache["B"], cache["T"]
    C, H = cfg["n_embd"], cfg["n_head"]
    hd = C // H
    BT = B * T
    bias = bool(cfg["bias"])
    tanh_form = bool(cfg["gelu_tanh"])
    G = {name: np.zeros(shape, dtype=dz.dtype) for name, shape in layout(cfg)}
    W = _lm_weight(cfg, P)
    dxf = _mm(ctr, dz, W)
    dW_lm = _mm(ctr, dz.T, cache["xf"])
    dx, G["lnf.w"], dbf = layernorm_bwd(dxf, cache["xhatf"], cache["rstdf"], P["lnf.w"])
    if bias:
        G["lnf.b"] = dbf
    for l in reversed(range(cfg["n_layer"])):
        p = f"h{l}."
        Lc = cache["layers"][l]
        # x_out = x_mid + GELU(u) W_fcproj^T + b
        dg = _mm(ctr, dx, P[p + "fcproj.w"])
        G[p + "fcproj.w"] = _mm(ctr, dx.T, Lc["g"])
        if bias:
            G[p + "fcproj.b"] = dx.sum(0)
        du = dg * gelu_grad(Lc["u"], tanh_form)
        da2 = _mm(ctr, du, P[p + "fc.w"])
        G[p + "fc.w"] = _mm(ctr, du.T, Lc["a2"])
        if bias:
            G[p + "fc.b"] = du.sum(0)
        dxl, G[p + "ln2.w"], db2 = layernorm_bwd(da2, Lc["xhat2"], Lc["rstd2"], P[p + "ln2.w"])
        if bias:
            G[p + "ln2.b"] = db2
        dx = dx + dxl
        # x_mid = x_in + y W_proj^T + b
        dy2 = _mm(ctr, dx, P[p + "proj.w"])
        G[p + "proj.w"] = _mm(ctr, dx.T, Lc["y2"])
        if bias:
            G[p + "proj.b"] = dx.sum(0)
        dy = dy2.reshape(B, T, H, hd).transpose(0, 2, 1, 3)
        dq = np.empty_like(Lc["q"])
        dk = np.empty_like(Lc["k"])
        dv = np.empty_like(Lc["v"])
        for b in range(B):
            dq[b], dk[b], dv[b] = attention_bwd(dy[b], Lc["q"][b], Lc["k"][b], Lc["v"][b],
                                                Lc["probs"][b], ctr)
        dqkv = np.concatenate([t.transpose(0, 2, 1, 3).reshape(BT, C) for t in (dq, dk, dv)], 1)
        da1 = _mm(ctr, dqkv, P[p + "qkv.w"])
        G[p + "qkv.w"] = _mm(ctr, dqkv.T, Lc["a1"])
        if bias:
            G[p + "qkv.b"] = dqkv.sum(0)
        dxl, G[p + "ln1.w"], db1 = layernorm_bwd(da1, Lc["xhat1"], Lc["rstd1"], P[p + "ln1.w"])
        if bias:
            G[p + "ln1.b"] = db1
        dx = dx + dxl
    # x0 = wte[idx] + wpe[t]
    dwte = np.zeros_like(P["wte"])
    np.add.at(dwte, cache["idx"].reshape(-1), dx)
    G["wpe"][:T] = dx.reshape(B, T, C).sum(0)
    if cfg["tied"]:
        G["wte"] = dW_lm + dwte
    else:
        G["wte"] = dwte
        G["lm_head.w"] = dW_lm
    return G


def logits(cfg, flat_params, idx, dtype=np.float64):
    P = unflatten(cfg, flat_params, dtype)
    z, _ = forward(cfg, P, np.asarray(idx))
    return z


def loss_rows(cfg, flat_params, idx, tgt, dtype=np.float64):
    """Per-token losses [B*T] for (idx, tgt) — each sequence's forward is independent."""
    z = logits(cfg, flat_params, idx, dtype)
    loss_r, _ = cross_entropy_fwd_bwd(z, np.asarray(tgt).reshape(-1), cfg["vocab_size"], z.shape[0])
    return loss_r


def loss_and_grads(cfg, flat_params, idx, tgt, dtype=np.float64, ctr=None):
    """Mean cross-entropy loss and the flat gradient vector (same layout as the parameters)."""
    idx = np.asarray(idx)
    tgt = np.asarray(tgt)
    P = unflatten(cfg, flat_params, dtype)
    z, cache = forward(cfg, P, idx, ctr)
    BT = z.shape[0]
    loss_r, dz = cross_entropy_fwd_bwd(z, tgt.reshape(-1), cfg["vocab_size"], BT)
    G = backward(cfg, P, cache, dz, ctr)
    return float(loss_r.mean()), flatten(cfg, G, dtype)


def grad_norm(flat_grads) -> float:
    g = np.asarray(flat_grads, dtype=np.float64)
    return float(np.sqrt(np.dot(g, g)))


def clip_scale(norm: float, max_norm: float) -> float:
    """Global-norm clipping factor (llm.c summary, "Proceso de entrenamiento")."""
    if max_norm <= 0.0 or norm <= max_norm:
        return 1.0
    return max_norm / norm


# --------------------------------------------------------------------------
# AdamW (nanochat "AdamW Fused Step")
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class AdamScalars:
    omb1: np.float32       # 1 - beta1
    omb2: np.float32       # 1 - beta2
    decay: np.float32      # 1 - lr * wd
    step_size: np.float32  # lr / (1 - beta1^t)
    sbc2: np.float32       # sqrt(1 - beta2^t)
    eps: np.float32
    scale: np.float32      # gradient multiplier (clipping)


def adamw_scalars(lr, beta1, beta2, eps, weight_decay, t, grad_scale=1.0) -> AdamScalars:
    """Each scalar in double precision from the hyper-parameters, rounded once to float32."""
    f = np.float32
    return AdamScalars(
        omb1=f(1.0 - beta1), omb2=f(1.0 - beta2), decay=f(1.0 - lr * weight_decay),
        step_size=f(lr / (1.0 - beta1 ** t)), sbc2=f(math.sqrt(1.0 - beta2 ** t)),
        eps=f(eps), scale=f(grad_scale))


def adamw_update(p, m, v, g, s: AdamScalars):
    """One AdamW step, float32, one rounded operation at a time:
    g*=scale; p*=decay; m+=omb1*(g-m); v+=omb2*(g*g-v); d=sqrt(v)/sbc2+eps; p-=step_size*(m/d).
    Returns new (p, m, v); the inputs are not modified."""
    f32 = np.float32
    p = np.asarray(p, f32)
    m = np.asarray(m, f32)
    v = np.asarray(v, f32)
    g = np.asarray(g, f32)
    g = g * s.scale
    p = p * s.decay
    m = m + s.omb1 * (g - m)
    v = v + s.omb2 * (g * g - v)
    d = np.sqrt(v) / s.sbc2 + s.eps
    p = p - s.step_size * (m / d)
    return p.astype(f32), m.astype(f32), v.astype(f32)


def bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even; NaN -> quiet NaN."""
    x = np.atleast_1d(np.asarray(x, np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[np.isnan(x)] = np.uint16(0x7FC0)
    return r


def bf16_round(x) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (returned as float32)."""
    return (bf16_bits(x).astype(np.uint32) << 16).view(np.float32)


def cosine_lr(t: int, max_lr: float, min_lr: float, warmup: int, decay_steps: int) -> float:
    """Learning rate of step t (1-based): a linear ramp to max_lr over `warmup`
    steps, then half a cosine period down to min_lr at `decay_steps`, then
    min_lr.  (Panthalia "Create a Plugin": helpers for cosine-annealed learning
    rates; nanoGPT README, "quick start": the rate decays until lr_decay_iters.
    The ramp and the half period are the plainest reading of "cosine annealing".)"""
    if warmup > 0 and t <= warmup:
        return max_lr * t / warmup
    if t >= decay_steps:
        return min_lr
    r = (t - warmup) / (decay_steps - warmup)
    return min_lr + 0.5 * (max_lr - min_lr) * (1.0 + math.cos(math.pi * r))


def train_steps(cfg, flat_params, batches, lrs, dtype=np.float64):
    """Several training steps with gradient accumulation (Panthalia "Create a
    Plugin": accumulations per step x examples per accumulation).
    batches[k] = list of (idx, tgt) micro-batches of step k + 1; lrs[k] its rate.
    Per step: the micro-batch gradients (each of a mean loss) are summed; the
    step's gradient is their mean, so AdamW gets grad_scale = clip / n where
    clip is the global-norm factor of that mean.  Returns dict(losses =
    per-step mean of the micro-batch losses, norms, p, m, v)."""
    p = np.asarray(flat_params, np.float32)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    losses, norms = [], []
    for k, micro in enumerate(batches):
        gsum = None
        lsum = 0.0
        for idx, tgt in micro:
            loss, g = loss_and_grads(cfg, p, idx, tgt, dtype)
            gsum = g if gsum is None else gsum + g
            lsum += loss
        n = len(micro)
        norm = grad_norm(gsum) / n
        scale = clip_scale(norm, cfg.get("clip", 0.0)) / n
        s = adamw_scalars(lrs[k], cfg["beta1"], cfg["beta2"], cfg["eps"], cfg["weight_decay"],
                          k + 1, scale)
        p, m, v = adamw_update(p, m, v, gsum.astype(np.float32), s)
        losses.append(lsum / n)
        norms.append(norm)
    return dict(losses=losses, norms=norms, p=p, m=m, v=v)


def step(cfg, flat_params, m, v, idx, tgt, t: int, dtype=np.float64):
    """One full training step: loss, gradients, global norm, clip, AdamW.
    Returns dict(loss, grads, norm, scale, p, m, v) with p/m/v float32."""
    loss, g = loss_and_grads(cfg, flat_params, idx, tgt, dtype)
    norm = grad_norm(g)
    scale = clip_scale(norm, cfg.get("clip", 0.0))
    s = adamw_scalars(cfg["lr"], cfg["beta1"], cfg["beta2"], cfg["eps"], cfg["weight_decay"],
                      t, scale)
    p1, m1, v1 = adamw_update(flat_params, m, v, g.astype(np.float32), s)
    return dict(loss=loss, grads=g, norm=norm, scale=scale, p=p1, m=m1, v=v1)


# --------------------------------------------------------------------------
# Muon for the 2-D block matrices, AdamW for the rest (nanochat
# "Optimierungsstrategien Muon und AdamW")
# --------------------------------------------------------------------------
# The page's "Polar Express" listing iterates over a coefficient table that the
# page does not print.  The plainest stand-in is the fixed quintic
# Newton-Schulz polynomial of the original Muon optimizer (K. Jordan et al.,
# "Muon: An optimizer for hidden layers in neural networks", 2024):
# p(s) = a s + b s^3 + c s^5 with these (a, b, c) at every iteration.
NS_COEFFS = (3.4445, -4.7750, 2.0315)


def muon_matrices(cfg):
    """Names of the tensors Muon updates: every per-layer Linear weight (attention
    and MLP matrices).  Embeddings, the lm_head and 0-D/1-D tensors go to AdamW
    (nanochat, "Verantwortlichkeiten und Design-Philosophie")."""
    return [n for n, s in layout(cfg) if len(s) == 2 and n not in ("wte", "wpe", "lm_head.w")]


def _r(x, bf16: bool):
    """Round to bfloat16 when computing in bfloat16 (PyTorch semantics: every
    op's result is stored in the tensor's dtype)."""
    return bf16_round(np.asarray(x, np.float64)).astype(np.float64) if bf16 else x


def orthogonalize(G, steps: int = 5, coeffs=NS_COEFFS, bf16: bool = True):
    """The page's orthogonalization listing ("Polar Express Details"):
    X = G in bf16; X /= ||X||_F * 1.01 + 1e-6; then `steps` times
      tall (rows > cols): A = X^T X, B = b A + c A A, X = a X + X B;
      otherwise (wide or square): A = X X^T, B = b A + c A A, X = a X + B X.
    (The wide branch of the listing uses B without defining it; it is the same
    polynomial in A as in the tall branch, which makes both branches apply
    p(s) = a s + b s^3 + c s^5 to every singular value.)
    With bf16=True every intermediate is rounded to bf16 as the listing's
    bf16 tensors would be; with bf16=False the iteration runs in float64."""
    X = _r(np.asarray(G, np.float64), bf16)
    n = _r(np.sqrt(np.sum(X * X)), bf16)
    den = _r(_r(n * 1.01, bf16) + 1e-6, bf16)
    X = _r(X / den, bf16)
    a, b, c = coeffs
    tall = X.shape[0] > X.shape[1]
    for _ in range(steps):
        A = _r(X.T @ X if tall else X @ X.T, bf16)
        AA = _r(A @ A, bf16)
        B = _r(_r(b * A, bf16) + _r(c * AA, bf16), bf16)
        XB = _r(X @ B if tall else B @ X, bf16)
        X = _r(_r(a * X, bf16) + XB, bf16)
    return X


def muon_momentum(g, buf, mu: float):
    """Momentum with the Nesterov look-ahead, in the lerp form the AdamW listing
    uses for its first moment: buf <- lerp(buf, g, 1 - mu); u = lerp(g, buf, mu).
    (The Muon pipeline diagram is missing from the page; this is the standard
    Muon momentum.)  float32, one rounded op at a time.  Returns (u, buf)."""
    f32 = np.float32
    g = np.asarray(g, f32)
    buf = np.asarray(buf, f32)
    buf = (buf + f32(1.0 - mu) * (g - buf)).astype(f32)
    u = (g + f32(mu) * (buf - g)).astype(f32)
    return u, buf


def muon_second_moment(X, v, beta2: float, eps: float = 1e-10):
    """The factored second moment (page: reduced row-wise for tall matrices,
    column-wise for wide ones).  Reading: one entry per index of the longer
    dimension (per row when rows > cols, else per column), the mean of X^2
    over the shorter dimension; v <- v + (1 - beta2) (s - v); each row (column)
    of X is divided by sqrt(v) + eps and the result rescaled to the Frobenius
    norm of X, so only the relative row (column) scales change.
    Returns (Y, v) in float64."""
    X = np.asarray(X, np.float64)
    tall = X.shape[0] > X.shape[1]
    s = np.mean(X * X, axis=1 if tall else 0)
    v = np.asarray(v, np.float64)
    v = v + (1.0 - beta2) * (s - v)
    d = np.sqrt(v) + eps
    Y = X / d[:, None] if tall else X / d[None, :]
    ny = np.sqrt(np.sum(Y * Y))
    if ny > 0:
        Y = Y * (np.sqrt(np.sum(X * X)) / ny)
    return Y, v


def cautious_update(p, Y, lr: float, wd: float):
    """The page's cautious update: mask = (Y * p >= 0); p -= lr * Y + lr * wd * p * mask
    (weight decay only where the update already pulls the parameter toward zero).
    float64."""
    p = np.asarray(p, np.float64)
    Y = np.asarray(Y, np.float64)
    mask = (Y * p) >= 0
    return p - (lr * Y + lr * wd * p * mask)


@dataclass(frozen=True)
class MuonHP:
    lr: float = 0.02
    momentum: float = 0.95
    beta2: float = 0.95
    weight_decay: float = 0.0
    ns_steps: int = 5
    eps: float = 1e-10


def muon_matrix_update(p, g, buf, v, hp: MuonHP, bf16: bool = True):
    """One Muon step of one matrix: momentum -> orthogonalization -> second
    moment -> cautious update (the page's four stages).  p, g, buf float32
    [rows, cols]; v float32 [max(rows, cols)].  Returns (p, buf, v) as float32."""
    u, buf = muon_momentum(g, buf, hp.momentum)
    X = orthogonalize(u, hp.ns_steps, NS_COEFFS, bf16)
    Y, v = muon_second_moment(X, v, hp.beta2, hp.eps)
    p = cautious_update(p, Y, hp.lr, hp.weight_decay)
    return p.astype(np.float32), buf, v.astype(np.float32)


def muon_hybrid_step(cfg, flat_params, m, v, flat_grads, adam_hp: dict, muon_hp: MuonHP,
                     t: int, grad_scale: float = 1.0, bf16: bool = True):
    """One optimizer step of the hybrid: Muon for `muon_matrices(cfg)`, AdamW
    (adamw_update) for every other tensor.  The gradients are multiplied by
    grad_scale first (float32).  For a Muon matrix the flat m slot holds its
    momentum buffer and the first max(rows, cols) entries of its v slot its
    second moment (the rest of that slot stays zero).  Returns (p, m, v) float32."""
    f32 = np.float32
    p = np.array(flat_params, f32)
    m = np.array(m, f32)
    v = np.array(v, f32)
    g = np.asarray(flat_grads, f32)
    muon = set(muon_matrices(cfg))
    s = adamw_scalars(adam_hp["lr"], adam_hp["beta1"], adam_hp["beta2"], adam_hp["eps"],
                      adam_hp["weight_decay"], t, grad_scale)
    off = 0
    for name, shape in layout(cfg):
        n = int(np.prod(shape))
        sl = slice(off, off + n)
        off += n
        if name in muon:
            L = max(shape)
            gs = (g[sl] * f32(grad_scale)).astype(f32).reshape(shape)
            pn, bn, vn = muon_matrix_update(p[sl].reshape(shape), gs, m[sl].reshape(shape),
                                            v[off - n:off - n + L], muon_hp, bf16)
            p[sl] = pn.reshape(-1)
            m[sl] = bn.reshape(-1)
            v[off - n:off - n + L] = vn
        else:
            p[sl], m[sl], v[sl] = adamw_update(p[sl], m[sl], v[sl], g[sl], s)
    return p, m, v


# --------------------------------------------------------------------------
# sampling (nanoGPT README, "sampling / inference": sample.py draws
# --num_samples continuations of --max_new_tokens tokens after a --start
# prompt; llm.c summary, "Sampling": unconditional / conditional sampling)
# --------------------------------------------------------------------------
def sample_token(z, V: int, temperature: float, top_k: int, u: float) -> int:
    """One draw from the logits z (entries >= V are padding and never drawn).
    temperature == 0: the argmax (the lowest index among equal maxima).
    Otherwise w = z[:V] / temperature; when 0 < top_k < V only entries >= the
    top_k-th largest w are kept (ties at the threshold kept);
    p_i = exp(w_i - max w) over the kept entries; the token is the smallest
    i with p_0 + ... + p_i > u * sum(p) (inverse CDF, u in [0, 1)).
    Readings: the pages name temperature-free "sampling"; temperature and
    top-k are the usual knobs of sample.py-style sampling and reduce to
    plain softmax sampling at temperature 1, top_k 0."""
    z = np.asarray(z, np.float64)[:V]
    if temperature == 0.0:
        return int(np.argmax(z))
    w = z / temperature
    keep = np.ones(V, bool)
    if 0 < top_k < V:
        thr = np.sort(w)[::-1][top_k - 1]
        keep = w >= thr
    m = w[keep].max()
    p = np.where(keep, np.exp(w - m), 0.0)
    c = np.cumsum(p)
    target = u * c[-1]
    i = int(np.searchsorted(c, target, side="right"))
    return min(i, int(np.flatnonzero(keep)[-1]))


def next_token_logits(cfg, flat_params, tokens, dtype=np.float64):
    """Logits of the last position of each row of tokens [B, T] from a full
    forward of the sequence so far (no cache: the definition a cached
    decoder must reproduce)."""
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    z = logits(cfg, flat_params, tokens, dtype)
    return z.reshape(B, T, -1)[:, -1, :]


def generate(cfg, flat_params, prompt, n_new: int, temperature: float, top_k: int, uniforms,
             dtype=np.float64):
    """Autoregressive continuation of prompt [B, T0] by n_new tokens; draw s of
    row b uses uniforms[b, s].  Reading: the sequence never exceeds
    block_size (no cropping of the context).  Returns [B, T0 + n_new]."""
    tokens = np.array(prompt, np.int32)
    B, T0 = tokens.shape
    if T0 + n_new > cfg["block_size"]:
        raise ValueError("prompt + new tokens exceed block_size")
    u = np.asarray(uniforms, np.float64).reshape(B, n_new)
    for s_ in range(n_new):
        z = next_token_logits(cfg, flat_params, tokens, dtype)
        nxt = np.array([sample_token(z[b], cfg["vocab_size"], temperature, top_k, u[b, s_])
                        for b in range(B)], np.int32)
        tokens = np.concatenate([tokens, nxt[:, None]], axis=1)
    return tokens


# --------------------------------------------------------------------------
# seeded initialisation (the weights N(0, 0.02) of the workload configs; gains
# 1, shifts and biases 0, padded vocabulary rows 0)
# --------------------------------------------------------------------------
_PHILOX_M = (0xD2511F53, 0xCD9E8D57)  # round multipliers
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)  # key increments (golden ratio, sqrt(3) - 1)


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel random
    numbers: as easy as 1, 2, 3", SC 2011).  ctr: [n, 4] counters, key: 2 words
    (uint32).  Each round multiplies words 0 and 2 by the two constants, and
    the new block is (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
    lo(M0 c0)); the key grows by the two increments before every round after
    the first.  Returns [n, 4] uint32."""
    mask = np.uint64(0xFFFFFFFF)
    c = np.asarray(ctr, dtype=np.uint64).reshape(-1, 4) & mask
    k0, k1 = (np.uint64(int(key[0]) & 0xFFFFFFFF), np.uint64(int(key[1]) & 0xFFFFFFFF))
    c0, c1, c2, c3 = c[:, 0], c[:, 1], c[:, 2], c[:, 3]
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(_PHILOX_W[0])) & mask
            k1 = (k1 + np.uint64(_PHILOX_W[1])) & mask
        p0 = np.uint64(_PHILOX_M[0]) * c0
        p1 = np.uint64(_PHILOX_M[1]) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & mask,
                          (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & mask)
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def philox_normals(begin: int, n: int, seed: int) -> np.ndarray:
    """Standard normals z[i] for flat indices i in [begin, begin + n), float64.
    Index i uses Philox block j = i // 4 (counter (j mod 2^32, j div 2^32, 0, 0),
    key (seed mod 2^32, seed div 2^32)); its words (x0, x1) give z[4j], z[4j+1]
    and (x2, x3) give z[4j+2], z[4j+3] by the Box-Muller transform (Box and
    Muller, 1958): u1 = (x + 1) / 2^32, u2 = x' / 2^32, r = sqrt(-2 ln u1),
    (r cos 2 pi u2, r sin 2 pi u2)."""
    if n <= 0:
        return np.zeros(0)
    j0, j1 = begin // 4, (begin + n - 1) // 4
    j = np.arange(j0, j1 + 1, dtype=np.uint64)
    ctr = np.stack([j & np.uint64(0xFFFFFFFF), j >> np.uint64(32),
                    np.zeros_like(j), np.zeros_like(j)], axis=1)
    x = philox4x32_10(ctr, (seed & 0xFFFFFFFF, seed >> 32)).astype(np.float64)
    z = np.empty((len(j), 4))
    for a, b in ((0, 1), (2, 3)):
        r = np.sqrt(-2.0 * np.log((x[:, a] + 1.0) / 4294967296.0))
        th = 2.0 * np.pi * (x[:, b] / 4294967296.0)
        z[:, a] = r * np.cos(th)
        z[:, b] = r * np.sin(th)
    z = z.reshape(-1)
    off = begin - 4 * j0
    return z[off:off + n]


def init_params(cfg, seed: int, std: float = 0.02) -> np.ndarray:
    """The flat float32 parameter vector of a seeded initialisation: every matrix
    and embedding entry is (float) (std * z[i]) with z the standard normal of
    its flat index i (philox_normals), except the padded vocabulary rows
    (>= vocab_size) of wte / lm_head, which are 0; LayerNorm gains are 1 and
    LayerNorm shifts and Linear biases 0."""
    V, out, off = cfg["vocab_size"], [], 0
    for name, shape in layout(cfg):
        n = int(np.prod(shape))
        if len(shape) == 2:
            a = (std * philox_normals(off, n, seed)).astype(np.float32)
            if name in ("wte", "lm_head.w"):
                a.reshape(shape)[V:] = 0.0
        elif name.endswith("ln1.w") or name.endswith("ln2.w") or name == "lnf.w":
            a = np.ones(n, np.float32)
        else:
            a = np.zeros(n, np.float32)
        out.append(a)
        off += n
    return np.concatenate(out)
