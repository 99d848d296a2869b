"""Single-kernel parity on the GPU through the C ABI, against the CPU oracle
(and plain numpy products as the definition of a matrix product)."""

import numpy as np
import pytest

import oracle
from decoder_only_gpt_amd import gpt, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gpt.lib()


def to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    return t.to(dtype)


def rounded(t):
    """The exact float values a device tensor holds, as float64 numpy."""
    return t.float().cpu().numpy().astype(np.float64)


# ------------------------------------------------------------------ AdamW
@pytest.mark.parametrize("t,scale", [(1, 1.0), (7, 0.37), (1000, 1.0)])
def test_adamw_bit_exact(t, scale):
    n = 1_000_003  # ragged tail
    rng = np.random.default_rng(t)
    p = rng.standard_normal(n).astype(np.float32)
    m, v, g = synth.adam_state(n, seed=t, scale=1e-3)
    special = np.array([0.0, -0.0, 1e-40, -3e-39, 1e-45, 65504.0, 1e-30], np.float32)
    p[:7], m[:7], v[:7] = special, special[::-1], np.abs(special)
    g[:7] = special[[3, 2, 1, 0, 6, 5, 4]]
    hp = gpt.AdamHP(1e-3, 0.9, 0.95, 1e-8, 0.01, scale, t)
    s = oracle.adamw_scalars(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t, scale)
    pr, mr, vr = oracle.adamw_update(p, m, v, g, s)
    dp, dm, dv, dg = (torch.from_numpy(x.copy()).cuda() for x in (p, m, v, g))
    sh = torch.empty(n, dtype=torch.int16, device="cuda")
    gpt.op_adamw(dp, dm, dv, dg, sh, hp)
    torch.cuda.synchronize()
    for got, ref in ((dp, pr), (dm, mr), (dv, vr)):
        assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(sh.cpu().numpy().view(np.uint16), oracle.bf16_bits(pr))


# ------------------------------------------------------------------ GEMM
def _operand(rows, K, trans, dtype, seed, gelu=False, tanh_form=False):
    """Device operand holding op(X) [rows, K]; returns (tensor, ld, exact values as [rows, K])."""
    ld = -(-rows // 8) * 8 if trans else -(-K // 8) * 8
    val = synth.normal((rows, K), seed, 1.0)
    if trans:
        store = np.zeros((K, ld), np.float32)
        store[:, :rows] = val.T
    else:
        store = np.zeros((rows, ld), np.float32)
        store[:, :K] = val
    dev = to_dev(store, dtype)
    exact = rounded(dev)
    exact = exact[:, :rows].T if trans else exact[:, :K]
    if gelu:
        exact = oracle.gelu(exact, tanh_form)
    return dev, ld, exact


CASES = [
    # M, N, K, a_trans, b_trans
    (200, 192, 136, 0, 0),      # forward layout, ragged M
    (130, 320, 64, 0, 1),       # dX layout (B stored [K, N])
    (96, 136, 203, 1, 1),       # dW layout, ragged K
    (256, 256, 4096, 1, 1),     # long K: split-K path
    (513, 64, 768, 0, 0),
]


@pytest.mark.parametrize("prec", [gpt.FP32, gpt.BF16])
@pytest.mark.parametrize("M,N,K,at,bt", CASES)
def test_gemm_layouts(prec, M, N, K, at, bt):
    dt = torch.bfloat16 if prec == gpt.BF16 else torch.float32
    A, lda, Ax = _operand(M, K, at, dt, 1)
    B, ldb, Bx = _operand(N, K, bt, dt, 2)
    ref = Ax @ Bx.T
    out = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    d = gpt.GemmDesc(precision=prec, M=M, N=N, K=K, A=A.data_ptr(), lda=lda, a_trans=at, a_rows=M,
                     a_kvalid=K, B=B.data_ptr(), ldb=ldb, b_trans=bt, b_rows=N, b_kvalid=K,
                     epilogue=gpt.EPI_F32, out=out.data_ptr(), ldo=N, workspace=ws.data_ptr(),
                     workspace_bytes=ws.numel())
    gpt.op_gemm(d)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err < 2e-5, err


WIDE_CASES = [
    # M, N, K, b_trans, epilogue: products whose 256 x 192 grid fills whole CU rounds
    (16344, 768, 520, 0, gpt.EPI_RESIDUAL),   # FC-projection / attention-projection forward
    (16344, 768, 1040, 1, gpt.EPI_STORE),     # FC / QKV input gradients
    (16344, 768, 264, 1, gpt.EPI_MUL),
    (16344, 768, 264, 1, gpt.EPI_DGELU),
    (16384, 2304, 136, 0, gpt.EPI_STORE),     # QKV forward (with bias)
]


@pytest.mark.parametrize("M,N,K,bt,epi", WIDE_CASES)
def test_gemm_wide_tiles(M, N, K, bt, epi):
    """The 256 x 192 tile plan (taken only at token-count M): ragged M and K;
    sampled rows, all columns, against exact values."""
    A, lda, Ax = _operand(M, K, 0, torch.bfloat16, 41)
    B, ldb, Bx = _operand(N, K, bt, torch.bfloat16, 42)
    bias = torch.from_numpy(synth.normal(N, 43, 0.5)).cuda()
    resid = torch.from_numpy(synth.normal((M, N), 44, 1.0)).cuda()
    aux = to_dev(synth.normal((M, N), 45, 1.5), torch.bfloat16)
    f32 = epi == gpt.EPI_RESIDUAL
    out = torch.zeros((M, N), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
    d = gpt.GemmDesc(precision=gpt.BF16, M=M, N=N, K=K, A=A.data_ptr(), lda=lda, a_trans=0, a_rows=M,
                     a_kvalid=K, B=B.data_ptr(), ldb=ldb, b_trans=bt, b_rows=N, b_kvalid=K,
                     epilogue=epi, gelu_tanh=1, out=out.data_ptr(), ldo=N)
    if epi in (gpt.EPI_STORE, gpt.EPI_RESIDUAL):
        d.bias = bias.data_ptr()
    if epi == gpt.EPI_RESIDUAL:
        d.resid = resid.data_ptr()
    if epi in (gpt.EPI_MUL, gpt.EPI_DGELU):
        d.aux, d.ldaux = aux.data_ptr(), N
    gpt.op_gemm(d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(46)
    rows = np.concatenate([rng.choice(M, 40, replace=False), [0, 255, 256, M - 1]])
    got = rounded(out)[rows]
    acc = Ax[rows] @ Bx.T
    bx = bias.cpu().numpy().astype(np.float64)
    if epi == gpt.EPI_RESIDUAL:
        ref = resid.cpu().numpy()[rows].astype(np.float64) + acc + bx
    elif epi == gpt.EPI_STORE:
        ref = acc + bx
    elif epi == gpt.EPI_MUL:
        ref = acc * rounded(aux)[rows]
    else:
        ref = acc * oracle.gelu_grad(rounded(aux)[rows], 1)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err < (2e-5 if f32 else 1e-2), err


@pytest.mark.parametrize("epi", [gpt.EPI_F32, gpt.EPI_F32_ACCUM])
def test_gemm_long_reduction_many_tiles(epi):
    """Weight-gradient layout with a long reduction over >= 256 output tiles of
    256 (the vocabulary weight gradient's plan: unsplit 256-tiles), ragged in
    M, N and K; sampled rows and columns against their exact values."""
    M, N, K = 4224, 3880, 2056
    A, lda, Ax = _operand(M, K, 1, torch.bfloat16, 31)
    B, ldb, Bx = _operand(N, K, 1, torch.bfloat16, 32)
    init = synth.normal((M, N), 33, 1.0).astype(np.float32)
    out = torch.from_numpy(init.copy()).cuda()
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    d = gpt.GemmDesc(precision=gpt.BF16, M=M, N=N, K=K, A=A.data_ptr(), lda=lda, a_trans=1, a_rows=M,
                     a_kvalid=K, B=B.data_ptr(), ldb=ldb, b_trans=1, b_rows=N, b_kvalid=K,
                     epilogue=epi, out=out.data_ptr(), ldo=N, workspace=ws.data_ptr(),
                     workspace_bytes=ws.numel())
    gpt.op_gemm(d)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rng = np.random.default_rng(34)
    rows = np.concatenate([rng.choice(M, 48, replace=False), [0, 255, 256, M - 1]])
    cols = np.concatenate([rng.choice(N, 48, replace=False), [0, 255, 256, N - 1]])
    ref = Ax[rows] @ Bx[cols].T + (init[np.ix_(rows, cols)] if epi == gpt.EPI_F32_ACCUM else 0.0)
    err = np.abs(got[np.ix_(rows, cols)] - ref).max() / np.abs(ref).max()
    assert err < 2e-5, err


ROUNDS_CASES = [
    # M, N, K, b_trans, epilogue: unsplit 256-tile plans of more than one round of
    # the 256 CUs
    (4000, 8144, 136, 0, gpt.EPI_GELU_PAIR),   # 512 tiles, ragged M / N
    (4000, 8144, 72, 1, gpt.EPI_MUL),          # input-gradient layout
    (4000, 8144, 200, 0, gpt.EPI_RESIDUAL),    # float output, ragged K
    (4000, 8144, 264, 1, gpt.EPI_DGELU),
    (16504, 16504, 64, 0, gpt.EPI_STORE),      # 4225 tiles (no XCD renumbering), one k-tile
]


@pytest.mark.parametrize("M,N,K,bt,epi", ROUNDS_CASES)
def test_gemm_many_rounds(M, N, K, bt, epi):
    """Unsplit 256-tile products over several rounds of the CUs, ragged in M,
    N and K; sampled rows (including the first and last of tiles), all
    columns, against exact values."""
    A, lda, Ax = _operand(M, K, 0, torch.bfloat16, 51)
    B, ldb, Bx = _operand(N, K, bt, torch.bfloat16, 52)
    bias = torch.from_numpy(synth.normal(N, 53, 0.5)).cuda()
    resid = torch.from_numpy(synth.normal((M, N), 54, 1.0)).cuda() if epi == gpt.EPI_RESIDUAL else None
    aux_in = to_dev(synth.normal((M, N), 55, 1.5), torch.bfloat16)
    f32 = epi == gpt.EPI_RESIDUAL
    out = torch.zeros((M, N), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
    aux = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    d = gpt.GemmDesc(precision=gpt.BF16, M=M, N=N, K=K, A=A.data_ptr(), lda=lda, a_trans=0, a_rows=M,
                     a_kvalid=K, B=B.data_ptr(), ldb=ldb, b_trans=bt, b_rows=N, b_kvalid=K,
                     epilogue=epi, gelu_tanh=1, out=out.data_ptr(), ldo=N)
    if epi in (gpt.EPI_STORE, gpt.EPI_RESIDUAL, gpt.EPI_GELU_PAIR):
        d.bias = bias.data_ptr()
    if epi == gpt.EPI_RESIDUAL:
        d.resid = resid.data_ptr()
    if epi == gpt.EPI_GELU_PAIR:
        d.aux, d.ldaux = aux.data_ptr(), N
    if epi in (gpt.EPI_MUL, gpt.EPI_DGELU):
        d.aux, d.ldaux = aux_in.data_ptr(), N
    gpt.op_gemm(d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(56)
    rows = np.unique(np.concatenate([rng.choice(M, 40, replace=False), [0, 255, 256, 3839, M - 1]]))
    rows_t = torch.from_numpy(rows).cuda()
    got = rounded(out[rows_t])
    acc = Ax[rows] @ Bx.T
    bx = bias.cpu().numpy().astype(np.float64)
    if epi == gpt.EPI_STORE:
        ref = acc + bx
    elif epi == gpt.EPI_RESIDUAL:
        ref = resid[rows_t].cpu().numpy().astype(np.float64) + acc + bx
    elif epi == gpt.EPI_MUL:
        ref = acc * rounded(aux_in[rows_t])
    elif epi == gpt.EPI_DGELU:
        ref = acc * oracle.gelu_grad(rounded(aux_in[rows_t]), 1)
    else:  # GELU pair: u = acc + bias rounded to bf16; out = GELU'(u), aux = GELU(u)
        u = oracle.bf16_round((acc + bx).astype(np.float32)).astype(np.float64)
        ref = oracle.gelu_grad(u, 1)
        g_ref = oracle.gelu(u, 1)
        g_err = np.abs(rounded(aux[rows_t]) - g_ref).max() / np.abs(g_ref).max()
        assert g_err < 1e-2, g_err
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err < (2e-5 if f32 else 1e-2), err


@pytest.mark.parametrize("prec", [gpt.FP32, gpt.BF16])
@pytest.mark.parametrize("epi", [gpt.EPI_STORE, gpt.EPI_RESIDUAL, gpt.EPI_GELU, gpt.EPI_DGELU,
                                 gpt.EPI_F32_ACCUM, gpt.EPI_GELU_PAIR, gpt.EPI_MUL])
@pytest.mark.parametrize("tanh_form", [0, 1])
@pytest.mark.parametrize("M,split", [(150, False), (16, True)])
def test_gemm_epilogues(prec, epi, tanh_form, M, split):
    """Every epilogue; M = 16 with a workspace is the few-row path (decode
    steps), split over K with the epilogue applied by the reduction."""
    dt = torch.bfloat16 if prec == gpt.BF16 else torch.float32
    N, K = 256, 192
    A, lda, Ax = _operand(M, K, 0, dt, 3, gelu=(epi == gpt.EPI_RESIDUAL), tanh_form=tanh_form)
    B, ldb, Bx = _operand(N, K, 0, dt, 4)
    if epi == gpt.EPI_RESIDUAL and prec == gpt.BF16:
        Ax = oracle.bf16_round(Ax.astype(np.float32)).astype(np.float64)  # GELU'd operand is bf16
    acc = Ax @ Bx.T
    bias = torch.from_numpy(synth.normal(N, 5, 0.5)).cuda()
    resid = torch.from_numpy(synth.normal((M, N), 6, 1.0)).cuda()
    aux_in = to_dev(synth.normal((M, N), 7, 1.5), dt)
    out_t = torch.float32 if epi in (gpt.EPI_RESIDUAL, gpt.EPI_F32_ACCUM) else dt
    out = torch.zeros((M, N), dtype=out_t, device="cuda")
    aux = torch.zeros((M, N), dtype=dt, device="cuda")
    if epi == gpt.EPI_F32_ACCUM:
        out.copy_(resid)
    d = gpt.GemmDesc(precision=prec, M=M, N=N, K=K, A=A.data_ptr(), lda=lda, a_trans=0, a_rows=M,
                     a_kvalid=K, a_gelu=int(epi == gpt.EPI_RESIDUAL), B=B.data_ptr(), ldb=ldb,
                     b_trans=0, b_rows=N, b_kvalid=K, epilogue=epi, gelu_tanh=tanh_form,
                     out=out.data_ptr(), ldo=N)
    if split:
        ws = torch.empty(32 * M * N * 4, dtype=torch.uint8, device="cuda")
        d.workspace, d.workspace_bytes = ws.data_ptr(), ws.numel()
    bx = bias.cpu().numpy().astype(np.float64)
    rx = resid.cpu().numpy().astype(np.float64)
    if epi in (gpt.EPI_STORE, gpt.EPI_GELU, gpt.EPI_RESIDUAL, gpt.EPI_GELU_PAIR):
        d.bias = bias.data_ptr()
    if epi == gpt.EPI_RESIDUAL:
        d.resid = resid.data_ptr()
    if epi in (gpt.EPI_GELU, gpt.EPI_GELU_PAIR):
        d.aux, d.ldaux = aux.data_ptr(), N
    if epi in (gpt.EPI_DGELU, gpt.EPI_MUL):
        d.aux, d.ldaux = aux_in.data_ptr(), N
    gpt.op_gemm(d)
    torch.cuda.synchronize()
    got = rounded(out)
    tol = 1e-2 if (prec == gpt.BF16 and out_t != torch.float32) else 2e-5
    if epi == gpt.EPI_RESIDUAL and prec == gpt.BF16:
        tol = 1e-3  # a GELU value may round to the neighbouring bf16 on either side
    if epi == gpt.EPI_STORE:
        ref = acc + bx
    elif epi == gpt.EPI_RESIDUAL:
        ref = rx + acc + bx
    elif epi == gpt.EPI_GELU:
        ref = acc + bx
        g_ref = oracle.gelu(got, tanh_form)   # GELU of the stored pre-activation
        g_err = np.abs(rounded(aux) - g_ref).max() / np.abs(g_ref).max()
        assert g_err < (1e-2 if prec == gpt.BF16 else 1e-6)
    elif epi == gpt.EPI_DGELU:
        ref = acc * oracle.gelu_grad(rounded(aux_in), tanh_form)
    elif epi == gpt.EPI_MUL:
        ref = acc * rounded(aux_in)
    elif epi == gpt.EPI_GELU_PAIR:
        # u = acc + bias rounded to the activation type; out = GELU'(u), aux = GELU(u)
        u = acc + bx
        if prec == gpt.BF16:
            u = oracle.bf16_round(u.astype(np.float32)).astype(np.float64)
        ref = oracle.gelu_grad(u, tanh_form)
        g_ref = oracle.gelu(u, tanh_form)
        g_err = np.abs(rounded(aux) - g_ref).max() / np.abs(g_ref).max()
        assert g_err < (1e-2 if prec == gpt.BF16 else 1e-5), g_err
    else:
        ref = rx + acc
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err < tol, err


def test_gemm_empty_and_padded_rows():
    """K = 0 runs the epilogue on zeros; B rows past b_rows read as zero."""
    M, N, K = 64, 128, 64
    A = torch.ones((M, K), dtype=torch.bfloat16, device="cuda")
    B = torch.ones((N, K), dtype=torch.bfloat16, device="cuda")
    out = torch.full((M, N), 3.0, device="cuda")
    d = gpt.GemmDesc(precision=gpt.BF16, M=M, N=N, K=K, A=A.data_ptr(), lda=K, a_rows=M, a_kvalid=K,
                     B=B.data_ptr(), ldb=K, b_rows=65, b_kvalid=K, epilogue=gpt.EPI_F32,
                     out=out.data_ptr(), ldo=N)
    gpt.op_gemm(d)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, :65] == K) and np.all(o[:, 65:] == 0)
    d.K = 0
    gpt.op_gemm(d)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 0)


# ------------------------------------------------------------------ attention
ATT = [  # B, T, H, hd, left
    (2, 1, 2, 64, -1),
    (2, 77, 2, 64, -1),
    (1, 300, 2, 64, -1),
    (1, 300, 2, 64, 100),
    (2, 200, 1, 32, 0),
    (1, 260, 2, 128, 64),
    (1, 129, 3, 128, -1),
    (1, 190, 2, 32, 17),
    (1, 600, 2, 64, 400),   # unmasked 128-row tiles inside a window, ragged end
    (1, 700, 1, 128, 300),
    (1, 512, 2, 32, -1),
]


def _attn_ref(qkv, dout, B, T, H, hd, left):
    C = H * hd
    q, k, v = (qkv[:, i * C:(i + 1) * C].reshape(B, T, H, hd).transpose(0, 2, 1, 3) for i in range(3))
    dy = dout.reshape(B, T, H, hd).transpose(0, 2, 1, 3)
    y = np.zeros((B, H, T, hd))
    lse = np.zeros((B, H, T))
    dq, dk, dv = np.zeros_like(y), np.zeros_like(y), np.zeros_like(y)
    for b in range(B):
        y[b], P = oracle.attention_fwd(q[b], k[b], v[b], left)
        S = (q[b] @ np.swapaxes(k[b], -1, -2)) / np.sqrt(hd)
        S = np.where(oracle.visible(T, left), S, -np.inf)
        mx = S.max(-1, keepdims=True)
        lse[b] = (mx + np.log(np.exp(S - mx).sum(-1, keepdims=True)))[..., 0]
        dq[b], dk[b], dv[b] = oracle.attention_bwd(dy[b], q[b], k[b], v[b], P)
    flat = lambda t: t.transpose(0, 2, 1, 3).reshape(B * T, C)
    return flat(y), lse, np.concatenate([flat(dq), flat(dk), flat(dv)], 1)


@pytest.mark.parametrize("prec", [gpt.FP32, gpt.BF16])
@pytest.mark.parametrize("B,T,H,hd,left", ATT)
def test_attention_fwd_bwd(prec, B, T, H, hd, left):
    dt = torch.bfloat16 if prec == gpt.BF16 else torch.float32
    C = H * hd
    qkv = to_dev(synth.normal((B * T, 3 * C), 11, 1.0), dt)
    dout = to_dev(synth.normal((B * T, C), 12, 1.0), dt)
    out = torch.zeros((B * T, C), dtype=dt, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    dqkv = torch.zeros((B * T, 3 * C), dtype=dt, device="cuda")
    ws = torch.zeros(2 * B * H * T + 1, dtype=torch.float32, device="cuda")
    gpt.op_attention_fwd(prec, B, T, H, hd, left, qkv, out, lse)
    gpt.op_attention_bwd(prec, B, T, H, hd, left, qkv, out, lse, dout, dqkv, ws)
    torch.cuda.synchronize()
    y_ref, lse_ref, dqkv_ref = _attn_ref(rounded(qkv), rounded(dout), B, T, H, hd, left)
    ftol = 1e-2 if prec == gpt.BF16 else 1e-5
    assert np.abs(rounded(out) - y_ref).max() / np.abs(y_ref).max() < ftol
    assert np.abs(lse.cpu().numpy() - lse_ref).max() < (2e-3 if prec == gpt.BF16 else 1e-5)
    g = rounded(dqkv)
    for i in range(3):
        a, r = g[:, i * C:(i + 1) * C], dqkv_ref[:, i * C:(i + 1) * C]
        if not np.abs(r).max():
            # exactly zero in real arithmetic (one visible key: dS = P (dP - D) = 0);
            # the device sees D from the rounded output, so only rounding noise remains
            assert np.abs(a).max() < 1e-4, (i, np.abs(a).max())
            continue
        err = np.abs(a - r).max() / np.abs(r).max()
        assert err < (3e-2 if prec == gpt.BF16 else 1e-4), (i, err)
        cos = (a * r).sum() / np.sqrt((a * a).sum() * (r * r).sum())
        assert cos > (0.9995 if prec == gpt.BF16 else 1 - 1e-9), (i, cos)


# ------------------------------------------------------------------ grouped GEMM
GROUP_CASES = [
    # reduction length K, products [(M, N)], epilogue
    (2048, [(64, 256), (256, 64), (64, 64), (192, 64)], gpt.EPI_F32),        # a small block's dW
    (3000, [(200, 136), (72, 512)], gpt.EPI_F32_ACCUM),                      # ragged tiles and K
    (2048, [(768, 3072), (3072, 768), (768, 768), (2304, 768)], gpt.EPI_F32),  # GPT-2 124M's block
    (1024, [(130, 72)], gpt.EPI_F32),                                         # a group of one
]


def _group_descs(K, shapes, epi, seed, trans_a=1):
    """Descriptors dW_i (+)= A_i^T-layout products for gpt_op_gemm_group, with
    the exact expected results; bias-gradient buffers (column sums of A_i,
    on every second product) with theirs."""
    ds, keep, refs, dbs, db_refs = [], [], [], [], []
    acc = epi == gpt.EPI_F32_ACCUM
    for i, (M, N) in enumerate(shapes):
        A, lda, Ax = _operand(M, K, trans_a if i == 0 else 1, torch.bfloat16, seed + 2 * i)
        B, ldb, Bx = _operand(N, K, 1, torch.bfloat16, seed + 2 * i + 1)
        init = synth.normal((M, N), seed + 50 + i, 1.0).astype(np.float32)
        out = torch.from_numpy(init.copy()).cuda()
        ref = Ax @ Bx.T + (init if acc else 0.0)
        ds.append(gpt.GemmDesc(precision=gpt.BF16, M=M, N=N, K=K, A=A.data_ptr(), lda=lda,
                               a_trans=trans_a if i == 0 else 1, a_rows=M, a_kvalid=K,
                               B=B.data_ptr(), ldb=ldb, b_trans=1, b_rows=N, b_kvalid=K,
                               epilogue=epi, out=out.data_ptr(), ldo=N))
        keep += [A, B, out]
        refs.append((out, ref))
        if i % 2 == 0:
            b0 = synth.normal((M,), seed + 80 + i, 1.0).astype(np.float32)
            db = torch.from_numpy(b0.copy()).cuda()
            dbs.append(db)
            db_refs.append((db, Ax.sum(axis=1) + (b0 if acc else 0.0)))
        else:
            dbs.append(None)
    return ds, keep, refs, dbs, db_refs


def _check_group(refs, db_refs, what):
    for out, ref in refs:
        err = np.abs(out.cpu().numpy() - ref).max() / np.abs(ref).max()
        assert err < 2e-5, (what, err)
    for db, ref in db_refs:  # fp32 sums of up to a few thousand bf16 values
        err = np.abs(db.cpu().numpy() - ref).max() / max(np.abs(ref).max(), 1.0)
        assert err < 2e-5, (what, "bias", err)


@pytest.mark.parametrize("K,shapes,epi", GROUP_CASES)
def test_gemm_group(K, shapes, epi):
    """A block's weight gradients in one grouped launch: every product matches
    its exact value (bf16 inputs, fp32 accumulation), for fresh and
    accumulated outputs, and so do the bias gradients the launch sums from
    its A tiles."""
    ds, keep, refs, dbs, db_refs = _group_descs(K, shapes, epi, seed=300)
    need = gpt.op_gemm_group_workspace([m for m, _ in shapes], [n for _, n in shapes], K)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for d in ds:
        d.workspace, d.workspace_bytes = ws.data_ptr(), ws.numel()
    gpt.op_gemm_group(ds, dbs)
    torch.cuda.synchronize()
    _check_group(refs, db_refs, "grouped")


def test_gemm_group_fallbacks():
    """A member the grouped kernel cannot take (row-major A) and a workspace
    too small for the partials both run product by product, with the same
    results; the group size is checked."""
    K, shapes = 1024, [(96, 128), (64, 256), (72, 64)]
    for trans_a, ws_bytes in ((0, 1 << 24), (1, 16)):
        ds, keep, refs, dbs, db_refs = _group_descs(K, shapes, gpt.EPI_F32, seed=400,
                                                    trans_a=trans_a)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        for d in ds:
            d.workspace, d.workspace_bytes = ws.data_ptr(), ws_bytes
        if trans_a == 0:  # a bias gradient needs a K-major A
            with pytest.raises(gpt.GptError):
                gpt.op_gemm_group(ds, dbs)
            dbs[0], db_refs = None, db_refs[1:]
        gpt.op_gemm_group(ds, dbs)
        torch.cuda.synchronize()
        _check_group(refs, db_refs, (trans_a, ws_bytes))
    with pytest.raises(gpt.GptError):
        gpt.op_gemm_group([])


# ------------------------------------------------------------------ batched GEMM
BATCH_CASES = [
    # batch, M, N, K, a_trans, b_trans, epilogue
    (3, 200, 136, 192, 0, 0, gpt.EPI_AXPBY),
    (3, 130, 256, 64, 0, 1, gpt.EPI_AXPBY),
    (3, 96, 136, 200, 1, 1, gpt.EPI_STORE),     # Gram layout, ragged K
    (4, 3072, 1024, 256, 0, 0, gpt.EPI_AXPBY),  # 256-tiles
    (4, 768, 768, 3072, 1, 1, gpt.EPI_STORE),   # the Gram product of a tall 3072 x 768 matrix
]


def _stacked(batch, rows, K, trans, dt, seed):
    """`batch` operands op(X_z) [rows, K] stored one after another; returns the
    device tensor, ld, byte stride and the exact values [batch, rows, K]."""
    ld = -(-rows // 8) * 8 if trans else -(-K // 8) * 8
    vals = np.stack([synth.normal((rows, K), seed + z, 1.0) for z in range(batch)])
    if trans:
        store = np.zeros((batch, K, ld), np.float32)
        store[:, :, :rows] = vals.transpose(0, 2, 1)
    else:
        store = np.zeros((batch, rows, ld), np.float32)
        store[:, :, :K] = vals
    dev = to_dev(store, dt)
    ex = rounded(dev)
    ex = ex[:, :, :rows].transpose(0, 2, 1) if trans else ex[:, :, :K]
    return dev, ld, dev[0].numel() * dev.element_size(), ex


@pytest.mark.parametrize("prec", [gpt.FP32, gpt.BF16])
@pytest.mark.parametrize("batch,M,N,K,at,bt,epi", BATCH_CASES)
def test_gemm_batched(prec, batch, M, N, K, at, bt, epi):
    """Batched products (the Newton-Schulz iteration's launches): every matrix
    of the batch against its own product, with the AXPBY epilogue
    out = alpha * acc + beta * aux.  At the GPT-2 124M Muon shapes the
    reference takes sampled rows of every matrix (all columns)."""
    dt = torch.bfloat16 if prec == gpt.BF16 else torch.float32
    A, lda, sa, Ax = _stacked(batch, M, K, at, dt, 10)
    B, ldb, sb, Bx = _stacked(batch, N, K, bt, dt, 20)
    aux = to_dev(np.stack([synth.normal((M, N), 30 + z, 1.0) for z in range(batch)]), dt)
    out = torch.zeros((batch, M, N), dtype=dt, device="cuda")
    alpha, beta = 2.0315, -4.775
    d = gpt.GemmDesc(precision=prec, M=M, N=N, K=K, A=A.data_ptr(), lda=lda, a_trans=at,
                     a_rows=M, a_kvalid=K, B=B.data_ptr(), ldb=ldb, b_trans=bt, b_rows=N,
                     b_kvalid=K, epilogue=epi, out=out.data_ptr(), ldo=N, alpha=alpha, beta=beta,
                     batch=batch, stride_a=sa, stride_b=sb, stride_out=M * N * out.element_size())
    if epi == gpt.EPI_AXPBY:
        d.aux, d.ldaux, d.stride_aux = aux.data_ptr(), N, M * N * aux.element_size()
    print(f"[gemm batched] prec={prec} batch={batch} {M}x{N}x{K} at={at} bt={bt} epi={epi}",
          flush=True)
    gpt.op_gemm(d)
    torch.cuda.synchronize()
    rows = np.arange(M)
    if M * N * K * batch > 1e9:
        rng = np.random.default_rng(M + N + K)
        rows = np.unique(np.concatenate([rng.choice(M, 40, replace=False), [0, M - 1]]))
    got = rounded(out)[:, rows]
    ref = np.matmul(Ax[:, rows], Bx.transpose(0, 2, 1))
    if epi == gpt.EPI_AXPBY:
        ref = alpha * ref + beta * rounded(aux)[:, rows]
    tol = 1e-2 if prec == gpt.BF16 else 2e-5
    for z in range(batch):
        err = np.abs(got[z] - ref[z]).max() / np.abs(ref[z]).max()
        assert err < tol, (z, err)
