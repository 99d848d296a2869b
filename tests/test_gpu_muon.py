"""The hybrid Muon + AdamW step on the GPU (through the C ABI) against the
oracle's muon_hybrid_step.

AdamW slices and the Muon momentum buffers: bit for bit (the same float32
operation sequence).  Muon parameter updates: fp32 within 1e-4 (relative
Frobenius, per matrix) of the float64 iteration.  bf16: the five quintic steps
amplify rounding in the directions of small singular values, so two bf16
evaluations that round at different points can differ by a few percent (more
for ill-conditioned gradients).  The bar is therefore relative to the page's
own bf16 listing: the device's update is no farther from the float64
iteration than 1.5x the oracle's bf16 iteration is (+1e-3), and has cosine
>= 0.99 with it.  The second moments follow the same split.  A forward after
the step checks that the bf16 weight copy was refreshed.
"""

import numpy as np
import pytest

import oracle
from decoder_only_gpt_amd import gpt, presets, synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gpt.lib()


CFGS = {
    "tiny": presets.preset("tiny"),
    "gpt2_s": presets.preset("gpt2_124m", vocab_size=500, padded_vocab=512, block_size=128,
                             n_layer=2, n_head=2, n_embd=128, mlp_hidden=512,
                             window_left=[-1, -1], B=2, T=64),
}
MUON = oracle.MuonHP(lr=0.02, momentum=0.95, beta2=0.95, weight_decay=0.1, ns_steps=5)


def _cos(a, b):
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
@pytest.mark.parametrize("name", ["tiny", "gpt2_s"])
def test_muon_hybrid_step_matches_oracle(name, prec):
    cfg = dict(CFGS[name], precision=prec)
    bf16 = prec == "bf16"
    p = synth.init_params(cfg, seed=8, perturb=True)
    n = p.size
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    model = gpt.Model(cfg)
    model.set_params(p)
    adam = dict(lr=cfg["lr"], beta1=cfg["beta1"], beta2=cfg["beta2"], eps=cfg["eps"],
                weight_decay=cfg["weight_decay"])
    mh = gpt.muon_hp(MUON.lr, MUON.momentum, MUON.beta2, MUON.weight_decay, MUON.eps,
                     MUON.ns_steps)
    muon = set(oracle.muon_matrices(cfg))
    for t, scale in ((1, 0.5), (2, 1.0)):
        g = synth.normal(n, seed=40 + t, scale=1e-2)
        print(f"[muon] {name} {prec} step {t}", flush=True)
        model.set_buffer(gpt.BUF_GRADS, g)
        model.muon_step(t, scale, mh)
        gp, gm, gv = model.params(), model.get_buffer(gpt.BUF_ADAM_M), model.get_buffer(gpt.BUF_ADAM_V)
        rp, rm, rv = oracle.muon_hybrid_step(cfg, p, m, v, g, adam, MUON, t, scale, bf16)
        if bf16:
            ep, _, ev = oracle.muon_hybrid_step(cfg, p, m, v, g, adam, MUON, t, scale, False)
        off = 0
        worst = 1.0
        for tname, shape in oracle.layout(cfg):
            k = int(np.prod(shape))
            sl = slice(off, off + k)
            if tname in muon:
                assert np.array_equal(gm[sl].view(np.uint32), rm[sl].view(np.uint32)), tname
                L = max(shape)
                d_got = gp[sl].astype(np.float64) - p[sl]
                d_ref = rp[sl].astype(np.float64) - p[sl]
                rel = np.linalg.norm(d_got - d_ref) / np.linalg.norm(d_ref)
                vg, vr = gv[off:off + L].astype(np.float64), rv[off:off + L].astype(np.float64)
                vrel = np.linalg.norm(vg - vr) / np.linalg.norm(vr)
                if bf16:
                    d_ex = ep[sl].astype(np.float64) - p[sl]
                    e_dev = np.linalg.norm(d_got - d_ex) / np.linalg.norm(d_ex)
                    e_or = np.linalg.norm(d_ref - d_ex) / np.linalg.norm(d_ex)
                    c = _cos(d_got, d_ex)
                    worst = min(worst, c)
                    assert e_dev <= 1.5 * e_or + 1e-3 and c >= 0.99, (tname, e_dev, e_or, c)
                    ve = ev[off:off + L].astype(np.float64)
                    v_dev = np.linalg.norm(vg - ve) / np.linalg.norm(ve)
                    v_or = np.linalg.norm(vr - ve) / np.linalg.norm(ve)
                    assert v_dev <= 1.5 * v_or + 1e-3, (tname, v_dev, v_or)
                else:
                    assert rel <= 1e-4, (tname, rel)
                    assert vrel <= 1e-4, (tname, vrel)
                assert not gv[off + L:off + k].any()
            else:
                for got, ref in ((gp, rp), (gm, rm), (gv, rv)):
                    assert np.array_equal(got[sl].view(np.uint32), ref[sl].view(np.uint32)), tname
            off += k
        print(f"[muon] {name} {prec} step {t}: worst update cosine vs float64 {worst:.5f}",
              flush=True)
        # continue both sides from the device state (the bf16 iteration is not bit-reproducible
        # across implementations, so the oracle takes the device's parameters)
        p, m, v = gp, gm, gv
    # the next forward reads the refreshed bf16 weight copy
    idx, tgt = synth.tokens(cfg, seed=9)
    model.forward(torch.from_numpy(idx.reshape(-1)).cuda(), torch.from_numpy(tgt.reshape(-1)).cuda())
    loss = model.loss()
    ref = oracle.loss_and_grads(cfg, p, idx, tgt)[0]
    assert abs(loss - ref) <= (2e-2 if bf16 else 1e-5) * ref


def test_muon_step_needs_backward_and_valid_hp():
    cfg = presets.preset("tiny")
    model = gpt.Model(cfg)
    with pytest.raises(gpt.GptError) as e:
        model.muon_step(1)
    assert e.value.code == gpt.E_STATE
    model.set_buffer(gpt.BUF_GRADS, np.zeros(model.n_params, np.float32))
    with pytest.raises(gpt.GptError) as e:
        model.muon_step(1, 1.0, gpt.muon_hp(momentum=1.0))
    assert e.value.code == gpt.E_INVALID
