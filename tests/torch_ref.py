"""An independent float64 PyTorch (CPU autograd) model of the same GPT.

Used only to pin the oracle's hand-derived backward against a library's
automatic differentiation.  It shares no code with the oracle: it uses
torch.nn.functional.layer_norm / gelu / cross_entropy and autograd.
"""

from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F


def _tensors(cfg, flat):
    C, Fh, Vp, Tb = cfg["n_embd"], cfg["mlp_hidden"], cfg["padded_vocab"], cfg["block_size"]
    names = [("wte", (Vp, C)), ("wpe", (Tb, C))]
    for l in range(cfg["n_layer"]):
        p = f"h{l}."
        for nm, shp, has_b, bshape in [("ln1", (C,), True, (C,)), ("qkv", (3 * C, C), True, (3 * C,)),
                                       ("proj", (C, C), True, (C,)), ("ln2", (C,), True, (C,)),
                                       ("fc", (Fh, C), True, (Fh,)), ("fcproj", (C, Fh), True, (C,))]:
            names.append((p + nm + ".w", shp))
            if cfg["bias"] and has_b:
                names.append((p + nm + ".b", bshape))
    names.append(("lnf.w", (C,)))
    if cfg["bias"]:
        names.append(("lnf.b", (C,)))
    if not cfg["tied"]:
        names.append(("lm_head.w", (Vp, C)))
    out, off = {}, 0
    flat = torch.as_tensor(np.asarray(flat, np.float64))
    for nm, shp in names:
        n = int(np.prod(shp))
        out[nm] = flat[off:off + n].reshape(shp).clone().requires_grad_(True)
        off += n
    assert off == flat.numel()
    return names, out


def loss_and_grads(cfg, flat, idx, tgt):
    names, P = _tensors(cfg, flat)
    idx = torch.as_tensor(np.asarray(idx, np.int64))
    tgt = torch.as_tensor(np.asarray(tgt, np.int64))
    B, T = idx.shape
    C, H = cfg["n_embd"], cfg["n_head"]
    hd = C // H
    eps = 1e-5
    gelu_mode = "tanh" if cfg["gelu_tanh"] else "none"
    x = P["wte"][idx] + P["wpe"][:T].unsqueeze(0)
    ii = torch.arange(T)[:, None]
    jj = torch.arange(T)[None, :]
    for l in range(cfg["n_layer"]):
        p = f"h{l}."
        left = cfg["window_left"][l]
        allowed = jj <= ii
        if left >= 0:
            allowed = allowed & (ii - jj <= left)
        a = F.layer_norm(x, (C,), P[p + "ln1.w"], P.get(p + "ln1.b"), eps)
        qkv = F.linear(a, P[p + "qkv.w"], P.get(p + "qkv.b"))
        q, k, v = qkv.split(C, dim=-1)
        q = q.view(B, T, H, hd).transpose(1, 2)
        k = k.view(B, T, H, hd).transpose(1, 2)
        v = v.view(B, T, H, hd).transpose(1, 2)
        att = (q @ k.transpose(-1, -2)) / math.sqrt(hd)
        att = att.masked_fill(~allowed, float("-inf"))
        y = torch.softmax(att, dim=-1) @ v
        y = y.transpose(1, 2).reshape(B, T, C)
        x = x + F.linear(y, P[p + "proj.w"], P.get(p + "proj.b"))
        a = F.layer_norm(x, (C,), P[p + "ln2.w"], P.get(p + "ln2.b"), eps)
        h = F.gelu(F.linear(a, P[p + "fc.w"], P.get(p + "fc.b")), approximate=gelu_mode)
        x = x + F.linear(h, P[p + "fcproj.w"], P.get(p + "fcproj.b"))
    x = F.layer_norm(x, (C,), P["lnf.w"], P.get("lnf.b"), eps)
    W = P["wte"] if cfg["tied"] else P["lm_head.w"]
    z = F.linear(x, W)[..., :cfg["vocab_size"]]
    loss = F.cross_entropy(z.reshape(-1, z.shape[-1]), tgt.reshape(-1))
    loss.backward()
    g = torch.cat([P[nm].grad.reshape(-1) for nm, _ in names])
    return float(loss.detach()), g.numpy()
