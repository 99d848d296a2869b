"""The allocation-free attention backward (gpt_op_attention_bwd_noalloc, static
device scratch) against gpt_op_attention_bwd with a caller workspace, through
the C ABI: bit for bit, on two calls in a row (the second smaller, so stale
scratch contents from the first are present), bf16 and fp32."""

import numpy as np
import pytest

from decoder_only_gpt_amd import gpt, synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gpt.lib()


def _inputs(prec, B, T, H, hd, left, seed):
    dt = torch.bfloat16 if prec == gpt.BF16 else torch.float32
    C = H * hd
    qkv = torch.from_numpy(synth.normal((B * T, 3 * C), seed, 1.0)).cuda().to(dt)
    out = torch.empty(B * T, C, dtype=dt, device="cuda")
    lse = torch.empty(B * H * T, dtype=torch.float32, device="cuda")
    gpt.op_attention_fwd(prec, B, T, H, hd, left, qkv, out, lse)
    dout = torch.from_numpy(synth.normal((B * T, C), seed + 1, 1.0)).cuda().to(dt)
    return qkv, out, lse, dout


@pytest.mark.parametrize("prec,hd", [(gpt.BF16, 64), (gpt.BF16, 128), (gpt.FP32, 64)])
def test_noalloc_matches_workspace_entry_point(prec, hd):
    shapes = [(4, 300, 3, -1), (2, 130, 2, 40)]  # second call smaller, windowed, ragged T
    for k, (B, T, H, left) in enumerate(shapes):
        print(f"noalloc case prec={prec} hd={hd} B={B} T={T} H={H} left={left}", flush=True)
        qkv, out, lse, dout = _inputs(prec, B, T, H, hd, left, 10 + k)
        ref = torch.zeros_like(qkv)
        ws = torch.empty(2 * B * H * T, dtype=torch.float32, device="cuda")
        gpt.op_attention_bwd(prec, B, T, H, hd, left, qkv, out, lse, dout, ref, ws)
        got = torch.full_like(qkv, 7.0)
        gpt.op_attention_bwd_noalloc(prec, B, T, H, hd, left, qkv, out, lse, dout, got)
        torch.cuda.synchronize()
        a = ref.view(torch.int16 if prec == gpt.BF16 else torch.int32).cpu().numpy()
        b = got.view(torch.int16 if prec == gpt.BF16 else torch.int32).cpu().numpy()
        assert np.array_equal(a, b)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    with pytest.raises(gpt.GptError) as e:
        gpt.op_attention_bwd_noalloc(gpt.BF16, 8, 2048, 65, 64, -1, None, None, None, None, None)
    assert e.value.code == gpt.E_INVALID
