"""Seeded parameter initialisation on the device (gpt_init) against the oracle's
Philox4x32-10 / Box-Muller definition, through the C ABI."""

import math

import numpy as np
import pytest

import oracle
from decoder_only_gpt_amd import gpt, presets, synth

from .test_gpu_step import gpu_cfgs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gpt.lib()


def _ulps(a, b):
    return np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))


@pytest.mark.parametrize("name,prec", [("tiny", "fp32"), ("gpt2_s", "bf16"), ("chat_s", "bf16")])
def test_device_init_matches_oracle(name, prec):
    """Every entry equals the oracle's float32 value (both sides evaluate
    Box-Muller in double; a last-bit difference of the libraries' log / sin /
    cos may move a rounding tie by one float32 ulp); exact zeros and ones
    where the definition puts them (padded vocabulary rows, biases, gains)."""
    cfg = presets.preset(name) if name == "tiny" else dict(gpu_cfgs()[name], precision=prec)
    m = gpt.Model(cfg, seed=7)
    got = m.params()
    ref = oracle.init_params(cfg, seed=7)
    special = (ref == 0) | (ref == 1)
    assert np.array_equal(got[special], ref[special])
    d = _ulps(got[~special], ref[~special])
    assert d.max() <= 1 and (d == 0).mean() > 0.9999
    assert not np.any(m.grads()) and not np.any(m.get_buffer(gpt.BUF_ADAM_M))


def test_device_init_seed_reproducible():
    cfg = gpu_cfgs()["chat_s"]
    a = gpt.Model(cfg, seed=3).params()
    b = gpt.Model(cfg, seed=3).params()
    c = gpt.Model(cfg, seed=4).params()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    normal = (a != 0) & (a != 1)
    assert np.all(a[normal] != c[normal])


def test_full_size_init_and_initial_loss():
    """GPT-2 124M shape: sampled windows of every tensor against the oracle's
    normals, padded vocabulary rows exactly 0, per-tensor mean and standard
    deviation within sampling error of N(0, 0.02), and the device loss of a
    Zipf batch at this init within the calibrated band above ln V."""
    cfg = presets.preset("gpt2_124m", B=2)
    m = gpt.Model(cfg, B=2, T=cfg["T"], seed=0)
    p = m.params()
    V, C = cfg["vocab_size"], cfg["n_embd"]
    off = 0
    for name, shape in oracle.layout(cfg):
        n = int(np.prod(shape))
        t = p[off:off + n]
        if len(shape) == 2:
            rows = t.reshape(shape)
            if name == "wte":
                assert not np.any(rows[V:])
                t = rows[:V].reshape(-1)
            for w0 in (0, len(t) // 2, len(t) - 4099):
                ref = (0.02 * oracle.philox_normals(off + w0, 4099, 0)).astype(np.float32)
                assert _ulps(t[w0:w0 + 4099], ref).max() <= 1, name
            x = t.astype(np.float64)
            assert abs(x.mean()) < 6 * 0.02 / math.sqrt(x.size), name
            assert abs(x.std() / 0.02 - 1) < 6 / math.sqrt(2 * x.size), name
        off += n
    idx, tgt = synth.tokens(cfg, B=2, T=cfg["T"], seed=1)
    m.forward(torch.from_numpy(idx.reshape(-1)).cuda(), torch.from_numpy(tgt.reshape(-1)).cuda())
    loss = m.loss()
    assert 0.0 <= loss - math.log(V) < 0.35, loss
