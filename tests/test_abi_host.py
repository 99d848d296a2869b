"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every symbol include/gpt.h declares, plans the documented sizes and rejects
bad configurations with the documented status codes."""

import ctypes
import json
import os
import re
import subprocess

import pytest

import oracle
from decoder_only_gpt_amd import gpt, presets

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = os.path.join(ROOT, "tests", "golden", "model_sizes.json")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gpt.LIB_PATH):
        from decoder_only_gpt_amd import build
        build.build()
    return gpt.lib()


def header_functions():
    src = open(os.path.join(ROOT, "include", "gpt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    declared = header_functions()
    assert set(declared) == set(gpt.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", gpt.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gpt_[a-z_0-9]+)$", out, flags=re.M))
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    for s in declared:
        assert hasattr(L, s)


@pytest.mark.parametrize("name", presets.ORDER)
def test_plan_matches_golden_sizes(L, name):
    cfg = presets.preset(name)
    g = json.load(open(GOLD))[name]
    s = gpt.plan(cfg, cfg["B"], cfg["T"])
    assert s.n_params == g["n_params"] == oracle.n_params(cfg)
    assert s.n_matmul_params == g["n_matmul"]
    assert s.flops_per_token == g["flops_per_token"]
    assert gpt.flops_per_token(cfg, g["T"]) == g["flops_per_token"]
    assert s.arena_bytes % 256 == 0 and s.arena_bytes > s.state_bytes >= 16 * s.n_params


def test_plan_fits_one_mi355x(L):
    """Every preset's whole training state + activations fits in 288 GB of HBM."""
    for name in presets.ORDER:
        cfg = presets.preset(name)
        s = gpt.plan(cfg, cfg["B"], cfg["T"])
        assert s.arena_bytes < 200e9


@pytest.mark.parametrize("field,value,code", [
    ("n_embd", 100, gpt.E_INVALID),           # not a multiple of 64 / n_head
    ("padded_vocab", 60, gpt.E_INVALID),      # below vocab_size
    ("n_head", 3, gpt.E_INVALID),             # 64 % 3 != 0
    ("mlp_hidden", 100, gpt.E_INVALID),
    ("precision", "fp16", None),              # maps to fp32 in the binding: fine
])
def test_config_errors(L, field, value, code):
    cfg = presets.preset("tiny")
    cfg[field] = value
    if code is None:
        gpt.plan(cfg, 4, 32)
        return
    with pytest.raises(gpt.GptError) as e:
        gpt.plan(cfg, 4, 32)
    assert e.value.code == code
    assert L.gpt_last_error().decode()


def test_shape_errors(L):
    cfg = presets.preset("tiny")
    with pytest.raises(gpt.GptError) as e:
        gpt.plan(cfg, 4, 33)  # T > block_size
    assert e.value.code == gpt.E_INVALID
    with pytest.raises(gpt.GptError) as e:
        gpt.plan(cfg, 0, 8)
    assert e.value.code == gpt.E_INVALID


def test_unsupported_head_dim_in_bf16(L):
    cfg = presets.preset("char", n_head=8)  # 384 / 8 = 48
    with pytest.raises(gpt.GptError) as e:
        gpt.plan(cfg, 2, 16)
    assert e.value.code == gpt.E_UNSUPPORTED
    cfg["precision"] = "fp32"
    gpt.plan(cfg, 2, 16)  # the fp32 path takes any head_dim <= 128


def test_null_arguments(L):
    s = gpt.Sizes()
    assert L.gpt_plan(None, 1, 1, ctypes.byref(s)) == gpt.E_INVALID
    assert L.gpt_forward(None, None, None, None) == gpt.E_INVALID
    assert L.gpt_backward(None, 0, None) == gpt.E_INVALID
    assert L.gpt_flops_per_token(None, 4) == 0.0
    hp = gpt.AdamHP(1e-3, 0.9, 0.95, 1e-8, 0.0, 1.0, 0)   # step_t = 0 is invalid
    assert L.gpt_op_adamw(0, None, None, None, None, None, ctypes.byref(hp), None) == gpt.E_INVALID
    d = gpt.GemmDesc()
    d.precision = 7
    assert L.gpt_op_gemm(ctypes.byref(d), None) == gpt.E_INVALID


def test_window_changes_only_attention_flops(L):
    cfg = presets.preset("nanochat_swa")
    full = dict(cfg, window_left=[-1] * 12)
    d = gpt.flops_per_token(full, 2048) - gpt.flops_per_token(cfg, 2048)
    assert d == 6 * 12 * 6 * 128 * (2048 - 512)


def test_binding_rejects_bad_token_tensors():
    """The binding hands the library only contiguous int32 CUDA tensors of B*T
    entries; anything else is refused before any device call (CPU only)."""
    import torch
    good = torch.zeros(8, dtype=torch.int32)
    with pytest.raises(TypeError):
        gpt.check_ids(torch.zeros(8, dtype=torch.int64), 8)
    with pytest.raises(TypeError):
        gpt.check_ids([0] * 8, 8)
    with pytest.raises(ValueError):
        gpt.check_ids(good, 8)  # not a CUDA tensor
    if torch.cuda.is_available():  # pragma: no cover - CPU suite
        return
    # shape / contiguity checks run after the device check; exercise them on
    # a tensor that claims to be on the device
    t = torch.zeros(16, dtype=torch.int32)
    import unittest.mock as um
    with um.patch.object(torch.Tensor, "is_cuda", new_callable=um.PropertyMock, return_value=True):
        gpt.check_ids(t[:8], 8)
        with pytest.raises(ValueError):
            gpt.check_ids(t, 8)
        with pytest.raises(ValueError):
            gpt.check_ids(t[::2], 8)
