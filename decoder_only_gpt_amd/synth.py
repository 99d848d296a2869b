"""Seeded synthetic inputs for the GPT training step.

This module only draws random numbers: token ids and initial weights.  It holds
none of the model's arithmetic, and both the device path and the CPU oracle are
fed from it, so they always see identical inputs.

Token ids: the character-level and GPT-2 datasets the pages train on are not
available, so each row is an i.i.d. Zipf draw over the real vocabulary,
p(k) proportional to (k+1)^-s, id 0 the most frequent, sampled by inverse CDF
from numpy's PCG64.  A row of T+1 ids gives the inputs row[:T] and the targets
row[1:] (the "input-target pairs" of the Panthalia plugin page, "Components").

Weights: every 2-D matrix and both embeddings ~ N(0, 0.02), LayerNorm gains 1,
shifts and biases 0, padded vocabulary rows exactly 0.  `perturb=True` adds
noise to gains, shifts and biases so that parity tests exercise every term.

The flat parameter order (a format both sides implement on their own) is: wte,
wpe, then per layer ln1.w, ln1.b, qkv.w, qkv.b, proj.w, proj.b, ln2.w, ln2.b,
fc.w, fc.b, fcproj.w, fcproj.b, then lnf.w, lnf.b, then lm_head.w when untied.
The ".b" entries exist only when bias=1; Linear weights are [out, in] row-major.
"""

from __future__ import annotations

import numpy as np


def _layout(cfg):
    """(name, shape, kind) in flat order; kind in matrix/embed/gain/shift."""
    C, F, Vp, Tb = cfg["n_embd"], cfg["mlp_hidden"], cfg["padded_vocab"], cfg["block_size"]
    out = [("wte", (Vp, C), "embed"), ("wpe", (Tb, C), "embed")]
    for l in range(cfg["n_layer"]):
        p = f"h{l}."
        out.append((p + "ln1.w", (C,), "gain"))
        if cfg["bias"]:
            out.append((p + "ln1.b", (C,), "shift"))
        out.append((p + "qkv.w", (3 * C, C), "matrix"))
        if cfg["bias"]:
            out.append((p + "qkv.b", (3 * C,), "shift"))
        out.append((p + "proj.w", (C, C), "matrix"))
        if cfg["bias"]:
            out.append((p + "proj.b", (C,), "shift"))
        out.append((p + "ln2.w", (C,), "gain"))
        if cfg["bias"]:
            out.append((p + "ln2.b", (C,), "shift"))
        out.append((p + "fc.w", (F, C), "matrix"))
        if cfg["bias"]:
            out.append((p + "fc.b", (F,), "shift"))
        out.append((p + "fcproj.w", (C, F), "matrix"))
        if cfg["bias"]:
            out.append((p + "fcproj.b", (C,), "shift"))
    out.append(("lnf.w", (C,), "gain"))
    if cfg["bias"]:
        out.append(("lnf.b", (C,), "shift"))
    if not cfg["tied"]:
        out.append(("lm_head.w", (Vp, C), "embed"))
    return out


def n_params(cfg) -> int:
    return int(sum(int(np.prod(s)) for _, s, _ in _layout(cfg)))


def init_params(cfg, seed: int = 0, std: float = 0.02, perturb: bool = False) -> np.ndarray:
    """Flat float32 parameter vector drawn from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    V = cfg["vocab_size"]
    chunks = []
    for name, shape, kind in _layout(cfg):
        n = int(np.prod(shape))
        if kind in ("matrix", "embed"):
            a = rng.standard_normal(n, dtype=np.float32) * np.float32(std)
            if name in ("wte", "lm_head.w"):
                a = a.reshape(shape)
                a[V:] = 0.0  # padded vocabulary rows start (and stay) at zero
                a = a.reshape(-1)
        elif kind == "gain":
            a = np.ones(n, np.float32)
            if perturb:
                a += rng.standard_normal(n, dtype=np.float32) * np.float32(0.1)
        else:
            a = np.zeros(n, np.float32)
            if perturb:
                a += rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)
        chunks.append(a.astype(np.float32, copy=False))
    return np.concatenate(chunks)


def zipf_cdf(V: int, s: float) -> np.ndarray:
    k = np.arange(1, V + 1, dtype=np.float64)
    w = k ** (-float(s))
    c = np.cumsum(w)
    return c / c[-1]


def tokens(cfg, B: int | None = None, T: int | None = None, seed: int = 1):
    """(idx, targets) int32 arrays of shape [B, T]: Zipf(s) ids, targets shifted by one."""
    B = cfg["B"] if B is None else B
    T = cfg["T"] if T is None else T
    rng = np.random.Generator(np.random.PCG64(seed))
    cdf = zipf_cdf(cfg["vocab_size"], cfg["zipf_s"])
    u = rng.random((B, T + 1))
    rows = np.searchsorted(cdf, u, side="right").astype(np.int32)
    np.minimum(rows, cfg["vocab_size"] - 1, out=rows)
    return np.ascontiguousarray(rows[:, :T]), np.ascontiguousarray(rows[:, 1:])


def adam_state(n: int, seed: int = 3, scale: float = 1e-3):
    """Random (m, v, g) float32 vectors for optimizer tests: m, g ~ N(0, scale), v = |N|^2 * scale^2."""
    rng = np.random.Generator(np.random.PCG64(seed))
    m = rng.standard_normal(n, dtype=np.float32) * np.float32(scale)
    v = np.square(rng.standard_normal(n, dtype=np.float32) * np.float32(scale))
    g = rng.standard_normal(n, dtype=np.float32) * np.float32(scale)
    return m, v, g


def normal(shape, seed: int, scale: float = 1.0, dtype=np.float32) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(dtype)
