"""Thin ctypes binding of libgptmi.so (include/gpt.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory (one arena tensor)
and the current stream.  If the library is missing this module raises; there
is no fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgptmi.so")

GPT_MAX_LAYERS = 128
OK, E_INVALID, E_STATE, E_HIP, E_NONFINITE, E_UNSUPPORTED = range(6)
FP32, BF16 = 0, 1
BUF_PARAMS, BUF_GRADS, BUF_ADAM_M, BUF_ADAM_V, BUF_LOSS_ROWS = range(5)
(EPI_STORE, EPI_RESIDUAL, EPI_GELU, EPI_DGELU, EPI_F32, EPI_F32_ACCUM, EPI_GELU_PAIR, EPI_MUL,
 EPI_AXPBY) = range(9)

# Every symbol include/gpt.h declares.
EXPORTS = [
    "gpt_plan", "gpt_flops_per_token", "gpt_init", "gpt_forward", "gpt_loss",
    "gpt_loss_device_ptr", "gpt_loss_async", "gpt_backward", "gpt_grad_norm", "gpt_adamw_step",
    "gpt_adamw_step_clipped", "gpt_muon_step",
    "gpt_get_buffer",
    "gpt_set_buffer", "gpt_destroy", "gpt_gen_plan", "gpt_gen_init", "gpt_gen_reset",
    "gpt_gen_set_graph",
    "gpt_gen_step", "gpt_gen_logits", "gpt_gen_sample", "gpt_generate", "gpt_gen_destroy",
    "gpt_last_error", "gpt_op_gemm", "gpt_op_gemm_group", "gpt_op_gemm_group_workspace",
    "gpt_op_attention_fwd", "gpt_op_attention_bwd", "gpt_op_attention_bwd_noalloc",
    "gpt_op_adamw", "gpt_profile_begin",
    "gpt_profile_end",
]
KERNEL_KINDS = ["gemm", "gemm_splitk", "attn_fwd", "attn_bwd", "layernorm", "cross_entropy",
                "embed", "bias_grad", "norm", "adamw"]
SITES = ["embed_fwd", "ln_fwd", "qkv_fwd", "attn_fwd", "proj_fwd", "fc_fwd", "fcproj_fwd",
         "lmhead_fwd", "cross_entropy", "lmhead_dx", "lmhead_dw", "ln_bwd", "fcproj_dx", "fcproj_dw",
         "fc_dx", "fc_dw", "proj_dx", "proj_dw", "attn_bwd", "qkv_dx", "qkv_dw", "bias_grad",
         "embed_bwd", "grad_norm", "adamw", "block_dw", "block_dw_reduce"]


GPT_E_NONFINITE = 4  # gpt_status: gradient norm is NaN or Inf


class GptError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"gpt status {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [
        ("vocab_size", ctypes.c_int32), ("padded_vocab", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("n_layer", ctypes.c_int32), ("n_head", ctypes.c_int32),
        ("n_embd", ctypes.c_int32), ("mlp_hidden", ctypes.c_int32), ("bias", ctypes.c_int32),
        ("tied_lm_head", ctypes.c_int32), ("gelu_tanh", ctypes.c_int32),
        ("precision", ctypes.c_int32), ("recompute_gelu", ctypes.c_int32),
        ("ln_eps", ctypes.c_float), ("window_left", ctypes.c_int32 * GPT_MAX_LAYERS),
    ]


class Sizes(ctypes.Structure):
    _fields_ = [
        ("n_params", ctypes.c_int64), ("n_matmul_params", ctypes.c_int64),
        ("flops_per_token", ctypes.c_double), ("arena_bytes", ctypes.c_int64),
        ("state_bytes", ctypes.c_int64), ("activation_bytes", ctypes.c_int64),
    ]


class AdamHP(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
        ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
        ("grad_scale", ctypes.c_double), ("step_t", ctypes.c_int64),
    ]


class KernelStats(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("ms", ctypes.c_double), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double)]


class MuonHP(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("momentum", ctypes.c_double), ("beta2", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("eps", ctypes.c_double),
                ("ns_steps", ctypes.c_int32)]


def muon_hp(lr=0.02, momentum=0.95, beta2=0.95, weight_decay=0.0, eps=1e-10, ns_steps=5) -> MuonHP:
    return MuonHP(lr, momentum, beta2, weight_decay, eps, ns_steps)


class GemmDesc(ctypes.Structure):
    _fields_ = [
        ("precision", ctypes.c_int32), ("M", ctypes.c_int32), ("N", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("a_trans", ctypes.c_int32),
        ("a_rows", ctypes.c_int32), ("a_kvalid", ctypes.c_int32), ("a_gelu", ctypes.c_int32),
        ("B", ctypes.c_void_p), ("ldb", ctypes.c_int64), ("b_trans", ctypes.c_int32),
        ("b_rows", ctypes.c_int32), ("b_kvalid", ctypes.c_int32), ("b_gelu", ctypes.c_int32),
        ("epilogue", ctypes.c_int32), ("gelu_tanh", ctypes.c_int32),
        ("bias", ctypes.c_void_p), ("resid", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("ldo", ctypes.c_int64),
        ("aux", ctypes.c_void_p), ("ldaux", ctypes.c_int64),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
        ("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("batch", ctypes.c_int32),
        ("stride_a", ctypes.c_int64), ("stride_b", ctypes.c_int64),
        ("stride_out", ctypes.c_int64), ("stride_aux", ctypes.c_int64),
    ]


_LIB = None


def lib():
    """Load libgptmi.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decoder_only_gpt_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "gpt_plan": ([ctypes.POINTER(Config), i32, i32, ctypes.POINTER(Sizes)], i32),
        "gpt_flops_per_token": ([ctypes.POINTER(Config), i32], ctypes.c_double),
        "gpt_init": ([ctypes.POINTER(Config), i32, i32, vp, i64, ctypes.c_uint64, vp,
                      ctypes.POINTER(vp)], i32),
        "gpt_forward": ([vp, vp, vp, vp], i32),
        "gpt_loss": ([vp, vp, ctypes.POINTER(ctypes.c_float)], i32),
        "gpt_loss_device_ptr": ([vp, ctypes.POINTER(vp)], i32),
        "gpt_backward": ([vp, i32, vp], i32),
        "gpt_grad_norm": ([vp, vp, ctypes.POINTER(ctypes.c_double)], i32),
        "gpt_adamw_step": ([vp, ctypes.POINTER(AdamHP), vp], i32),
        "gpt_adamw_step_clipped": ([vp, ctypes.POINTER(AdamHP), i32, ctypes.c_double, vp, vp], i32),
        "gpt_loss_async": ([vp, vp, vp], i32),
        "gpt_muon_step": ([vp, ctypes.POINTER(AdamHP), ctypes.POINTER(MuonHP), vp], i32),
        "gpt_gen_plan": ([vp, i32, i32, ctypes.POINTER(i64)], i32),
        "gpt_gen_init": ([vp, i32, i32, vp, i64, vp, ctypes.POINTER(vp)], i32),
        "gpt_gen_reset": ([vp], i32),
        "gpt_gen_set_graph": ([vp, i32], i32),
        "gpt_gen_step": ([vp, vp, vp], i32),
        "gpt_gen_logits": ([vp, vp, ctypes.POINTER(i64), vp], i32),
        "gpt_gen_sample": ([vp, ctypes.c_float, i32, vp, i64, vp, vp], i32),
        "gpt_generate": ([vp, vp, i32, i32, ctypes.c_float, i32, vp, vp, vp], i32),
        "gpt_gen_destroy": ([vp], i32),
        "gpt_get_buffer": ([vp, i32, vp, i32, vp], i32),
        "gpt_set_buffer": ([vp, i32, vp, i32, vp], i32),
        "gpt_destroy": ([vp], i32),
        "gpt_last_error": ([], ctypes.c_char_p),
        "gpt_op_gemm": ([ctypes.POINTER(GemmDesc), vp], i32),
        "gpt_op_gemm_group": ([ctypes.POINTER(GemmDesc), vp, i32, vp], i32),
        "gpt_op_gemm_group_workspace": ([ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                         i32, i32], i64),
        "gpt_op_attention_fwd": ([i32, i32, i32, i32, i32, i32, vp, vp, vp, vp], i32),
        "gpt_op_attention_bwd": ([i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp], i32),
        "gpt_op_attention_bwd_noalloc": ([i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp],
                                         i32),
        "gpt_op_adamw": ([i64, vp, vp, vp, vp, vp, ctypes.POINTER(AdamHP), vp], i32),
        "gpt_profile_begin": ([vp], i32),
        "gpt_profile_end": ([vp, vp, ctypes.POINTER(KernelStats), ctypes.POINTER(KernelStats)], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _LIB = L
    return L


def _check(code):
    if code != OK:
        raise GptError(code, lib().gpt_last_error().decode())


def make_config(cfg: dict) -> Config:
    c = Config()
    c.vocab_size = cfg["vocab_size"]
    c.padded_vocab = cfg["padded_vocab"]
    c.block_size = cfg["block_size"]
    c.n_layer = cfg["n_layer"]
    c.n_head = cfg["n_head"]
    c.n_embd = cfg["n_embd"]
    c.mlp_hidden = cfg["mlp_hidden"]
    c.bias = int(cfg["bias"])
    c.tied_lm_head = int(cfg["tied"])
    c.gelu_tanh = int(cfg["gelu_tanh"])
    c.precision = BF16 if cfg["precision"] == "bf16" else FP32
    c.recompute_gelu = int(cfg.get("recompute_gelu", 0))
    c.ln_eps = float(cfg.get("ln_eps", 1e-5))
    w = cfg["window_left"]
    if len(w) > GPT_MAX_LAYERS:
        raise ValueError("too many layers")
    for i, v in enumerate(w):
        c.window_left[i] = int(v)
    return c


def plan(cfg: dict, B: int, T: int) -> Sizes:
    s = Sizes()
    _check(lib().gpt_plan(ctypes.byref(make_config(cfg)), B, T, ctypes.byref(s)))
    return s


def flops_per_token(cfg: dict, T: int) -> float:
    return lib().gpt_flops_per_token(ctypes.byref(make_config(cfg)), T)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def check_ids(t, n: int, what: str = "idx"):
    """Token ids handed to the library must be a contiguous int32 CUDA tensor
    of n entries (the kernels read n int32 values at its address)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if t.dtype != torch.int32:
        raise TypeError(f"{what} must be int32, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{what} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() != n:
        raise ValueError(f"{what} must have {n} entries, got {t.numel()}")


def adam_hp(cfg: dict, t: int, grad_scale: float = 1.0, lr: float | None = None) -> AdamHP:
    return AdamHP(cfg["lr"] if lr is None else lr, cfg["beta1"], cfg["beta2"], cfg["eps"],
                  cfg["weight_decay"], grad_scale, t)


class Model:
    """One model bound to a device arena; methods map 1:1 onto the C ABI."""

    def __init__(self, cfg: dict, B: int | None = None, T: int | None = None, seed: int = 0):
        import torch
        self.cfg = dict(cfg)
        self.B = cfg["B"] if B is None else B
        self.T = cfg["T"] if T is None else T
        self.sizes = plan(cfg, self.B, self.T)
        self.n_params = int(self.sizes.n_params)
        self.arena = torch.empty(int(self.sizes.arena_bytes), dtype=torch.uint8, device="cuda")
        h = ctypes.c_void_p()
        self._c = make_config(cfg)
        _check(lib().gpt_init(ctypes.byref(self._c), self.B, self.T,
                              ctypes.c_void_p(self.arena.data_ptr()), int(self.sizes.arena_bytes),
                              ctypes.c_uint64(int(seed)), _stream(), ctypes.byref(h)))
        self.h = h
        self.step_t = 0

    def __del__(self):
        h = getattr(self, "h", None)
        if h is not None and _LIB is not None:
            _LIB.gpt_destroy(h)
            self.h = None

    # ---- buffers
    def set_buffer(self, which: int, data):
        import torch
        if isinstance(data, torch.Tensor):
            assert data.is_cuda and data.dtype == torch.float32 and data.numel() == self.n_params
            data = data.contiguous()
            _check(lib().gpt_set_buffer(self.h, which, ctypes.c_void_p(data.data_ptr()), 1, _stream()))
            torch.cuda.current_stream().synchronize()
        else:
            a = np.ascontiguousarray(data, dtype=np.float32)
            assert a.size == self.n_params
            _check(lib().gpt_set_buffer(self.h, which, a.ctypes.data_as(ctypes.c_void_p), 0, _stream()))

    def get_buffer(self, which: int) -> np.ndarray:
        n = self.B * self.T if which == BUF_LOSS_ROWS else self.n_params
        out = np.empty(n, np.float32)
        _check(lib().gpt_get_buffer(self.h, which, out.ctypes.data_as(ctypes.c_void_p), 0, _stream()))
        return out

    def set_params(self, p):
        self.set_buffer(BUF_PARAMS, p)

    def params(self):
        return self.get_buffer(BUF_PARAMS)

    def grads(self):
        return self.get_buffer(BUF_GRADS)

    # ---- the step
    def forward(self, idx, tgt=None):
        n = self.B * self.T
        check_ids(idx, n, "idx")
        if tgt is not None:
            check_ids(tgt, n, "tgt")
        self._idx, self._tgt = idx, tgt  # keep the device tensors alive
        _check(lib().gpt_forward(self.h, ctypes.c_void_p(idx.data_ptr()),
                                 None if tgt is None else ctypes.c_void_p(tgt.data_ptr()), _stream()))

    def loss(self) -> float:
        out = ctypes.c_float()
        _check(lib().gpt_loss(self.h, _stream(), ctypes.byref(out)))
        return float(out.value)

    def backward(self, accumulate: int = 0):
        _check(lib().gpt_backward(self.h, int(accumulate), _stream()))

    def grad_norm(self) -> float:
        out = ctypes.c_double()
        _check(lib().gpt_grad_norm(self.h, _stream(), ctypes.byref(out)))
        return float(out.value)

    def adamw_step(self, t: int, grad_scale: float = 1.0, lr: float | None = None):
        hp = adam_hp(self.cfg, t, grad_scale, lr)
        _check(lib().gpt_adamw_step(self.h, ctypes.byref(hp), _stream()))

    def _pinned(self):
        """Page-locked host slots for the asynchronous read-backs: loss (float32)
        and {norm, grad_scale} (float64)."""
        if getattr(self, "_pin", None) is None:
            import torch
            self._pin = (torch.zeros(1, dtype=torch.float32, pin_memory=True),
                         torch.zeros(2, dtype=torch.float64, pin_memory=True))
        return self._pin

    def loss_async(self):
        """Enqueue the loss copy into the page-locked slot (read it after a sync)."""
        pl, _ = self._pinned()
        _check(lib().gpt_loss_async(self.h, ctypes.c_void_p(pl.data_ptr()), _stream()))

    def adamw_step_clipped(self, t: int, max_norm: float, n_micro: int = 1,
                           lr: float | None = None):
        """Device-side norm, clip and AdamW; {norm, grad_scale} land in the
        page-locked slot (read them after a sync)."""
        _, pn = self._pinned()
        hp = adam_hp(self.cfg, t, 1.0, lr)
        _check(lib().gpt_adamw_step_clipped(self.h, ctypes.byref(hp), int(n_micro), float(max_norm),
                                            ctypes.c_void_p(pn.data_ptr()), _stream()))

    def muon_step(self, t: int, grad_scale: float = 1.0, muon: MuonHP | None = None,
                  lr: float | None = None):
        """Muon on the per-layer Linear weights, AdamW (lr, t, grad_scale) on the rest."""
        hp = adam_hp(self.cfg, t, grad_scale, lr)
        mh = muon if muon is not None else muon_hp()
        _check(lib().gpt_muon_step(self.h, ctypes.byref(hp), ctypes.byref(mh), _stream()))

    def profile_begin(self):
        _check(lib().gpt_profile_begin(self.h))

    def profile_end(self):
        """(per kernel kind, per call site) dicts of launches / ms / flops / bytes."""
        arr = (KernelStats * len(KERNEL_KINDS))()
        sites = (KernelStats * len(SITES))()
        _check(lib().gpt_profile_end(self.h, _stream(), arr, sites))
        conv = lambda names, a: {k: dict(launches=int(x.launches), ms=x.ms, flops=x.flops,
                                          bytes=x.bytes) for k, x in zip(names, a)}
        return conv(KERNEL_KINDS, arr), conv(SITES, sites)

    def train_step(self, idx, tgt) -> dict:
        """forward -> loss -> backward -> (norm, clip) -> AdamW; returns loss/norm/scale.
        Everything is enqueued before any host wait: the loss and the norm /
        clip scale come back through asynchronous copies, read after one sync
        at the end (while AdamW still runs on the model's side stream)."""
        import torch
        self.forward(idx, tgt)
        self.loss_async()
        self.backward(0)
        t = self.step_t + 1
        clip = float(self.cfg.get("clip", 0.0) or 0.0)
        if clip > 0.0:
            self.adamw_step_clipped(t, clip)
        else:
            self.adamw_step(t, 1.0)
        torch.cuda.current_stream().synchronize()
        pl, pn = self._pinned()
        loss = float(pl[0])
        norm, scale = (float(pn[0]), float(pn[1])) if clip > 0.0 else (None, 1.0)
        # An update the device skipped does not count as an optimizer step.
        if math.isnan(loss):  # the library's mark for an out-of-range token id
            raise GptError(E_INVALID, "loss is NaN: a token id or target is outside [0, vocab_size) "
                                      "(the update was skipped) or the loss diverged")
        if norm is not None and not math.isfinite(norm):
            raise GptError(GPT_E_NONFINITE, f"gradient norm is not finite ({norm}); no update")
        self.step_t = t
        return dict(loss=loss, norm=norm, scale=scale)


class Generator:
    """Key/value-cache generation on a model's weights (B sequences of up to
    Tmax tokens); methods map 1:1 onto the gpt_gen_* entry points."""

    def __init__(self, model: Model, B: int, Tmax: int, graph: bool = True):
        import torch
        self.model, self.B, self.Tmax = model, B, Tmax
        n = ctypes.c_int64()
        _check(lib().gpt_gen_plan(model.h, B, Tmax, ctypes.byref(n)))
        self.arena = torch.empty(int(n.value), dtype=torch.uint8, device="cuda")
        h = ctypes.c_void_p()
        _check(lib().gpt_gen_init(model.h, B, Tmax, ctypes.c_void_p(self.arena.data_ptr()),
                                  int(n.value), _stream(), ctypes.byref(h)))
        self.h = h
        self._keep = []
        _check(lib().gpt_gen_set_graph(self.h, int(bool(graph))))

    def __del__(self):
        h = getattr(self, "h", None)
        if h is not None and _LIB is not None:
            _LIB.gpt_gen_destroy(h)
            self.h = None

    def reset(self):
        _check(lib().gpt_gen_reset(self.h))

    def step(self, tokens):
        """tokens: device int32 tensor [B]."""
        self._keep = [tokens]
        _check(lib().gpt_gen_step(self.h, ctypes.c_void_p(tokens.data_ptr()), _stream()))

    def logits(self) -> np.ndarray:
        """Last step's logits as float32 [B, vocab_size]."""
        bf16 = self.model.cfg["precision"] == "bf16"
        Vq = -(-self.model.cfg["padded_vocab"] // 64) * 64
        raw = np.empty(self.B * Vq, np.uint16 if bf16 else np.float32)
        ld = ctypes.c_int64()
        _check(lib().gpt_gen_logits(self.h, raw.ctypes.data_as(ctypes.c_void_p), ctypes.byref(ld),
                                    _stream()))
        z = (raw.astype(np.uint32) << 16).view(np.float32) if bf16 else raw
        return z.reshape(self.B, int(ld.value))[:, :self.model.cfg["vocab_size"]]

    def sample(self, temperature: float, top_k: int, u=None, u_stride: int = 1):
        """Device int32 tensor [B] of drawn tokens; u: device float tensor (or None for greedy)."""
        import torch
        out = torch.empty(self.B, dtype=torch.int32, device="cuda")
        _check(lib().gpt_gen_sample(self.h, float(temperature), int(top_k),
                                    None if u is None else ctypes.c_void_p(u.data_ptr()),
                                    int(u_stride), ctypes.c_void_p(out.data_ptr()), _stream()))
        return out

    def generate(self, prompt, n_new: int, temperature: float, top_k: int, uniforms=None):
        """prompt: device int32 [B, T0]; uniforms: device float [B, n_new] (or None for
        greedy).  Returns the device int32 tensor [B, T0 + n_new]."""
        import torch
        B, T0 = prompt.shape
        out = torch.empty((B, T0 + n_new), dtype=torch.int32, device="cuda")
        _check(lib().gpt_generate(self.h, ctypes.c_void_p(prompt.data_ptr()), int(T0), int(n_new),
                                  float(temperature), int(top_k),
                                  None if uniforms is None else ctypes.c_void_p(uniforms.data_ptr()),
                                  ctypes.c_void_p(out.data_ptr()), _stream()))
        return out


# ---------------------------------------------------------------- single ops
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def op_gemm(desc: GemmDesc):
    _check(lib().gpt_op_gemm(ctypes.byref(desc), _stream()))


def op_gemm_group(descs, bias_grads=None):
    """gpt_op_gemm_group over a list of GemmDesc (1..4); bias_grads: None or a
    list of float32 device tensors (or None) receiving the column sums of A."""
    arr = (GemmDesc * len(descs))(*descs)
    db = None
    if bias_grads is not None:
        db = (ctypes.c_void_p * len(descs))(*[None if t is None else t.data_ptr() for t in bias_grads])
    _check(lib().gpt_op_gemm_group(arr, db, len(descs), _stream()))


def op_gemm_group_workspace(Ms, Ns, K: int) -> int:
    n = len(Ms)
    return int(lib().gpt_op_gemm_group_workspace((ctypes.c_int32 * n)(*Ms), (ctypes.c_int32 * n)(*Ns),
                                                 n, int(K)))


def op_attention_fwd(precision, B, T, H, hd, left, qkv, out, lse):
    _check(lib().gpt_op_attention_fwd(precision, B, T, H, hd, left, _ptr(qkv), _ptr(out), _ptr(lse),
                                      _stream()))


def op_attention_bwd(precision, B, T, H, hd, left, qkv, out, lse, dout, dqkv, workspace):
    _check(lib().gpt_op_attention_bwd(precision, B, T, H, hd, left, _ptr(qkv), _ptr(out), _ptr(lse),
                                      _ptr(dout), _ptr(dqkv), _ptr(workspace), _stream()))


def op_attention_bwd_noalloc(precision, B, T, H, hd, left, qkv, out, lse, dout, dqkv):
    _check(lib().gpt_op_attention_bwd_noalloc(precision, B, T, H, hd, left, _ptr(qkv), _ptr(out),
                                              _ptr(lse), _ptr(dout), _ptr(dqkv), _stream()))


def op_adamw(p, m, v, g, shadow, hp: AdamHP):
    _check(lib().gpt_op_adamw(p.numel(), _ptr(p), _ptr(m), _ptr(v), _ptr(g), _ptr(shadow),
                              ctypes.byref(hp), _stream()))
