"""Generation with a key/value cache on the GPU (through the C ABI) against
the oracle, which recomputes a full forward of the sequence so far for every
new token.

* decode logits: fp32 within 1e-4 of the largest |logit| of the oracle's
  float64 forward at every position; bf16 within 3e-2 of it (bf16 weights,
  activations and cache);
* the sampler: temperature 0 gives the argmax of the device logits (lowest
  index on ties); otherwise the token is a valid inverse-CDF draw for u from
  the device logits -- the oracle's float64 cumulative sums put u*total
  between the token's lower and upper cumulative sums (up to 1e-5 relative,
  the float32 summation of the device) -- and lies in the top-k set;
* fp32 generation (greedy and sampled) equals the oracle's token for token;
  bf16 generation equals the composition of the device's own steps and draws.
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
                             window_left=[-1, -1], B=3, T=64),
    "chat_s": presets.preset("nanochat_swa", vocab_size=300, padded_vocab=300, block_size=160,
                             n_layer=2, n_head=1, n_embd=128, mlp_hidden=256,
                             window_left=[20, -1], B=2, T=64),
    # wider than the bf16 decode products fold the LayerNorm into (1024), and an
    # FC projection long enough (K = 2048) for 16 waves per workgroup
    "wide_s": presets.preset("gpt2_124m", vocab_size=200, padded_vocab=208, block_size=64,
                             n_layer=1, n_head=9, n_embd=1152, mlp_hidden=2048,
                             window_left=[-1], B=2, T=16),
}


def _setup(name, prec, seed=0):
    cfg = dict(CFGS[name], precision=prec)
    p = synth.init_params(cfg, seed=seed, perturb=True)
    m = gpt.Model(cfg, B=1, T=8)
    m.set_params(p)
    return cfg, p, m


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
@pytest.mark.parametrize("name", ["tiny", "gpt2_s", "chat_s", "wide_s"])
def test_decode_logits_match_full_forward(name, prec):
    cfg, p, m = _setup(name, prec)
    B, T = 3, {"tiny": 32, "wide_s": 16}.get(name, 48)
    seq, _ = synth.tokens(cfg, B=B, T=T, seed=11)
    g = gpt.Generator(m, B, T)
    tol = 3e-2 if prec == "bf16" else 1e-4
    print(f"[gen] logits {name} {prec} B={B} T={T}", flush=True)
    worst = 0.0
    for t in range(T):
        g.step(_dev(seq[:, t]))
        z = g.logits()
        ref = oracle.next_token_logits(cfg, p, seq[:, :t + 1])[:, :cfg["vocab_size"]]
        err = np.abs(z - ref).max() / np.abs(ref).max()
        worst = max(worst, err)
        assert err <= tol, (t, err)
    print(f"[gen] {name} {prec} worst logit error {worst:.2e}", flush=True)


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
@pytest.mark.parametrize("B", [1, 20])
def test_decode_logits_row_groups(prec, B):
    """The bf16 decode products take rows in groups of 16: one sequence (15
    rows of the group stand in for row 0), and 20 (the second group, rows
    16..19, runs with a ragged tail)."""
    cfg, p, m = _setup("chat_s", prec, seed=3)
    T = 24
    seq, _ = synth.tokens(cfg, B=B, T=T, seed=15)
    g = gpt.Generator(m, B, T)
    tol = 3e-2 if prec == "bf16" else 1e-4
    print(f"[gen] logits chat_s {prec} B={B} T={T}", flush=True)
    for t in range(T):
        g.step(_dev(seq[:, t]))
        z = g.logits()
        ref = oracle.next_token_logits(cfg, p, seq[:, :t + 1])[:, :cfg["vocab_size"]]
        err = np.abs(z - ref).max(axis=1) / np.abs(ref).max(axis=1)
        assert err.max() <= tol, (B, t, int(err.argmax()), float(err.max()))


def _valid_draw(z, V, temperature, top_k, u, tok):
    w = np.asarray(z, np.float64)[:V] / temperature
    keep = np.ones(V, bool)
    if 0 < top_k < V:
        keep = w >= np.sort(w)[::-1][top_k - 1]
    assert keep[tok], "token outside the top-k set"
    p = np.where(keep, np.exp(w - w[keep].max()), 0.0)
    c = np.cumsum(p)
    target = u * c[-1]
    lo = c[tok - 1] if tok > 0 else 0.0
    assert lo <= target * (1 + 1e-5) + 1e-12 and c[tok] >= target * (1 - 1e-5), (tok, lo, c[tok],
                                                                                    target)


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
@pytest.mark.parametrize("name", ["gpt2_s", "chat_s"])
def test_sampler_draws_are_valid(name, prec):
    cfg, p, m = _setup(name, prec, seed=2)
    B = 3
    V = cfg["vocab_size"]
    seq, _ = synth.tokens(cfg, B=B, T=5, seed=12)
    g = gpt.Generator(m, B, 8)
    for t in range(5):
        g.step(_dev(seq[:, t]))
    z = g.logits().astype(np.float64)
    # greedy: the argmax of the device logits
    tok = g.sample(0.0, 0).cpu().numpy()
    for b in range(B):
        assert tok[b] == int(np.argmax(z[b])), b
    rng = np.random.default_rng(3)
    cases = [(1.0, 0), (0.7, 5), (1.3, 50), (1.0, V - 1), (1.0, V), (0.05, 0), (2.0, 1)]
    for temperature, top_k in cases:
        for u in [0.0, 0.999999, *rng.random(6)]:
            ud = torch.full((B,), float(u), dtype=torch.float32, device="cuda")
            tok = g.sample(temperature, top_k, ud).cpu().numpy()
            for b in range(B):
                _valid_draw(z[b], V, temperature, top_k, float(np.float32(u)), int(tok[b]))
                if top_k == 1:
                    assert tok[b] == int(np.argmax(z[b]))


@pytest.mark.parametrize("temperature,top_k", [(0.0, 0), (0.8, 20), (1.0, 0)])
@pytest.mark.parametrize("name", ["tiny", "gpt2_s", "chat_s"])
def test_fp32_generation_matches_oracle(name, temperature, top_k):
    cfg, p, m = _setup(name, "fp32", seed=4)
    B, T0 = 2, 6
    n_new = min(30, cfg["block_size"] - T0)
    prompt, _ = synth.tokens(cfg, B=B, T=T0, seed=13)
    u = np.random.default_rng(7).random((B, n_new)).astype(np.float32)
    g = gpt.Generator(m, B, T0 + n_new)
    print(f"[gen] generate {name} fp32 t={temperature} k={top_k}", flush=True)
    out = g.generate(_dev(prompt), n_new, temperature, top_k,
                     torch.from_numpy(u).cuda()).cpu().numpy()
    ref = oracle.generate(cfg, p, prompt, n_new, temperature, top_k, u.astype(np.float64))
    assert np.array_equal(out, ref), np.argwhere(out != ref)[:4]


@pytest.mark.parametrize("name", ["gpt2_s", "chat_s"])
def test_bf16_generation_is_its_steps_and_draws(name):
    cfg, p, m = _setup(name, "bf16", seed=5)
    B, T0, n_new = 3, 4, 20
    prompt, _ = synth.tokens(cfg, B=B, T=T0, seed=14)
    u = torch.from_numpy(np.random.default_rng(8).random((B, n_new)).astype(np.float32)).cuda()
    g = gpt.Generator(m, B, T0 + n_new)
    out = g.generate(_dev(prompt), n_new, 0.9, 30, u).cpu().numpy()
    assert np.array_equal(out[:, :T0], prompt)
    g.reset()
    for t in range(T0 + n_new - 1):
        g.step(_dev(out[:, t]))
        if t >= T0 - 1:
            k = t - T0 + 1
            tok = g.sample(0.9, 30, u[:, k:], n_new).cpu().numpy()
            assert np.array_equal(tok, out[:, t + 1]), t
    # and the run is reproducible
    again = g.generate(_dev(prompt), n_new, 0.9, 30, u).cpu().numpy()
    assert np.array_equal(again, out)


def test_generation_errors():
    cfg, p, m = _setup("tiny", "fp32")
    g = gpt.Generator(m, 2, 4)
    with pytest.raises(gpt.GptError) as e:
        g.sample(0.0, 0)
    assert e.value.code == gpt.E_STATE
    tok = _dev(np.zeros(2))
    for _ in range(4):
        g.step(tok)
    with pytest.raises(gpt.GptError) as e:
        g.step(tok)
    assert e.value.code == gpt.E_INVALID
    g.reset()
    g.step(tok)
    with pytest.raises(gpt.GptError) as e:
        g.generate(_dev(np.zeros((2, 3))), 2, 0.0, 0)
    assert e.value.code == gpt.E_INVALID
    with pytest.raises(gpt.GptError):
        gpt.Generator(m, 1, cfg["block_size"] + 1)


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
@pytest.mark.parametrize("name", ["gpt2_s", "chat_s"])
def test_graph_replay_equals_eager_steps(name, prec):
    """Decode steps replayed from the captured graph give the same logits, bit
    for bit, as the same steps launched one kernel at a time, at every
    position; with eager work and synchronisations between the replays, a
    reset in the middle, and whole-sequence generation on both paths."""
    cfg, p, m = _setup(name, prec)
    B, T = 3, 24
    seq, _ = synth.tokens(cfg, B=B, T=T, seed=13)
    gg = gpt.Generator(m, B, T, graph=True)
    ge = gpt.Generator(m, B, T, graph=False)
    for rnd in range(2):  # the second round after a reset of both
        for t in range(T):
            tok = _dev(seq[:, t])
            gg.step(tok)
            ze = None
            if t % 5 == 0:
                torch.cuda.synchronize()
            ge.step(tok)
            zg, ze = gg.logits(), ge.logits()
            assert np.array_equal(zg.view(np.uint32) if zg.dtype == np.float32 else zg,
                                  ze.view(np.uint32) if ze.dtype == np.float32 else ze), (rnd, t)
        gg.reset()
        ge.reset()
    prompt = _dev(seq[:, :6])
    u = torch.from_numpy(np.random.default_rng(3).random((B, 10), dtype=np.float32)).cuda()
    og = gg.generate(prompt, 10, 0.8, 20, u)
    oe = ge.generate(prompt, 10, 0.8, 20, u)
    assert torch.equal(og, oe)
