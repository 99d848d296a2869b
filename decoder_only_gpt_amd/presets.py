"""Named workloads of the decoder-only GPT training step (plain data, no arithmetic).

Each preset fixes the model shape, the micro-batch, the precision and the AdamW
hyper-parameters of one workload.  The shapes follow the configurations the
nanoGPT README describes ("quick start": 6 layers, 6 heads, 384 channels,
context 256 for the character-level run; "reproducing GPT-2" for the 124M
model), the llm.c summary ("Modelo 350M", "-r" recompute flag) and the
nanochat architecture page ("FLOPs-Berechnung im Detail": per-layer
(left, right) attention windows).

Fields
------
vocab_size     real vocabulary (softmax runs over these columns only)
padded_vocab   rows of the token-embedding / lm_head matrix (>= vocab_size)
block_size     maximum context
n_layer, n_head, n_embd, mlp_hidden
bias           1: LayerNorm shifts and Linear biases exist; 0: LayerNorm gain only
tied           1: lm_head reuses the token embedding; 0: separate lm_head matrix
gelu_tanh      1: tanh-approximated GELU; 0: exact erf GELU
precision      "fp32" or "bf16"
recompute_gelu 1: GELU(u) is not stored, it is recomputed where it is read
window_left    per-layer left window (-1 = full causal)
B, T           micro-batch and sequence length of one step
zipf_s         exponent of the synthetic token distribution
lr, beta1, beta2, eps, weight_decay, clip   AdamW / clipping hyper-parameters
"""

from __future__ import annotations

import copy

_BASE_ADAMW = dict(beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.01)

PRESETS = {
    # Tiny fp32 GPT: the parity workload the oracle finishes in well under a second.
    "tiny": dict(
        vocab_size=65, padded_vocab=65, block_size=32, n_layer=2, n_head=2, n_embd=64,
        mlp_hidden=256, bias=0, tied=1, gelu_tanh=0, precision="fp32", recompute_gelu=0,
        window_left=[-1, -1], B=4, T=32, zipf_s=1.1, lr=1e-3, clip=0.0, **_BASE_ADAMW),
    # Character-level GPT (nanoGPT README, quick start), bf16 activations.
    "char": dict(
        vocab_size=65, padded_vocab=65, block_size=256, n_layer=6, n_head=6, n_embd=384,
        mlp_hidden=1536, bias=0, tied=1, gelu_tanh=0, precision="bf16", recompute_gelu=0,
        window_left=[-1] * 6, B=64, T=256, zipf_s=1.1, lr=1e-4, clip=0.0, **_BASE_ADAMW),
    # GPT-2 124M shape, LayerNorm and Linear biases, tanh GELU, clip at 1.0.
    "gpt2_124m": dict(
        vocab_size=50257, padded_vocab=50304, block_size=1024, n_layer=12, n_head=12,
        n_embd=768, mlp_hidden=3072, bias=1, tied=1, gelu_tanh=1, precision="bf16",
        recompute_gelu=0, window_left=[-1] * 12, B=16, T=1024, zipf_s=1.05, lr=1e-4,
        clip=1.0, **_BASE_ADAMW),
    # GPT-2 350M shape with GELU recompute in the backward pass.
    "gpt2_350m": dict(
        vocab_size=50257, padded_vocab=50304, block_size=1024, n_layer=24, n_head=16,
        n_embd=1024, mlp_hidden=4096, bias=1, tied=1, gelu_tanh=1, precision="bf16",
        recompute_gelu=1, window_left=[-1] * 24, B=8, T=1024, zipf_s=1.05, lr=1e-4,
        clip=0.0, **_BASE_ADAMW),
    # nanochat-style: head_dim 128, untied lm_head, sliding window 512 on even layers.
    "nanochat_swa": dict(
        vocab_size=65536, padded_vocab=65536, block_size=2048, n_layer=12, n_head=6,
        n_embd=768, mlp_hidden=3072, bias=0, tied=0, gelu_tanh=0, precision="bf16",
        recompute_gelu=0, window_left=[512 if l % 2 == 0 else -1 for l in range(12)],
        B=8, T=2048, zipf_s=1.05, lr=1e-4, clip=0.0, **_BASE_ADAMW),
}

ORDER = ["tiny", "char", "gpt2_124m", "gpt2_350m", "nanochat_swa"]


def preset(name: str, **overrides) -> dict:
    """A deep copy of preset `name` with `overrides` applied."""
    cfg = copy.deepcopy(PRESETS[name])
    for k, v in overrides.items():
        if k not in cfg:
            raise KeyError(f"unknown preset field {k!r}")
        cfg[k] = v
    if len(cfg["window_left"]) != cfg["n_layer"]:
        raise ValueError("window_left needs one entry per layer")
    return cfg
