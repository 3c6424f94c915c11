"""Per-kernel parity on the GPU, through the C ABI, against the oracle's
per-operation functions (NumPy), on seeded inputs.

Sizes span several tiles plus ragged tails; the large cases use the real
7B-shaped dimensions and compare sampled rows.
"""
import numpy as np
import pytest

import oracle
from oracle import decoder as D

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch


def _mt():
    from layer_streamed_amd import mt
    return mt


def bf16_dev(a):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(torch.bfloat16)


def to_np(t):
    return t.float().cpu().numpy()


def rel_fro(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-30))


def _rand(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


GEMM_CASES = [
    # layout, M, N, K  (ragged M/N tails, K not a multiple of 64)
    (0, 300, 200, 264), (1, 300, 200, 264), (2, 296, 200, 264),
    (0, 256, 512, 256), (1, 256, 256, 1024), (2, 1024, 256, 256),
    (0, 128, 128, 64), (1, 8, 8, 8), (2, 8, 8, 8),
    # direct-to-LDS tiles with ragged M and N (a partial last 16-column
    # group takes the per-element epilogue) and, for NT, an odd ldc (no
    # 16-byte epilogue at all)
    (0, 300, 200, 256), (1, 300, 200, 256), (2, 296, 200, 256), (0, 300, 203, 256),
]


@pytest.mark.parametrize("layout,M,N,K", GEMM_CASES)
@pytest.mark.parametrize("epi", [0, 1, 2, 3])
def test_gemm_layouts_and_epilogues(layout, M, N, K, epi):
    torch, mt = _torch(), _mt()
    rng = np.random.default_rng(100 + layout * 7 + epi)
    a = oracle.bf16_round(_rand(rng, (K, M) if layout == 2 else (M, K)))
    b = oracle.bf16_round(_rand(rng, (N, K) if layout == 0 else (K, N)))
    A, B = bf16_dev(a), bf16_dev(b)
    af = a.astype(np.float64)
    bf = b.astype(np.float64)
    ref = (af.T if layout == 2 else af) @ (bf.T if layout == 0 else bf)
    r = None
    if epi == 3:
        r = oracle.bf16_round(_rand(rng, (M, N)))
        ref = ref + r
    if epi in (1, 2):
        Cm = torch.zeros((M, N), device="cuda", dtype=torch.float32)
        if epi == 2:
            init = _rand(rng, (M, N))
            Cm.copy_(torch.from_numpy(init))
            ref = ref + init
    else:
        Cm = torch.zeros((M, N), device="cuda", dtype=torch.bfloat16)
    lda = M if layout == 2 else K
    ldb = K if layout == 0 else N
    mt.gemm(layout, epi, M, N, K, A, lda, B, ldb, Cm, N, R=None if r is None else bf16_dev(r), ldr=N)
    torch.cuda.synchronize()
    out = to_np(Cm)
    tol = 1e-5 if epi in (1, 2) else 5e-3
    assert rel_fro(out, ref) < tol
    if epi not in (1, 2):
        np.testing.assert_allclose(out, ref, rtol=1e-2, atol=1e-2 * np.abs(ref).max())


@pytest.mark.parametrize("layout,M,N,K", [(0, 300, 200, 264), (1, 300, 200, 256), (2, 296, 200, 256),
                                           (0, 256, 512, 256), (0, 300, 203, 256)])
def test_gemm_bf16_store_is_rne_of_the_fp32_result(layout, M, N, K):
    """The bf16 epilogues round in the device (gfx950's packed conversion):
    the same product stored as fp32 (same accumulation, same order) and then
    rounded to nearest even by the oracle must give the bf16 store bit for
    bit, plain and with the residual added in fp32 first."""
    torch, mt = _torch(), _mt()
    rng = np.random.default_rng(700 + layout)
    a = oracle.bf16_round(_rand(rng, (K, M) if layout == 2 else (M, K)))
    b = oracle.bf16_round(_rand(rng, (N, K) if layout == 0 else (K, N)))
    r = oracle.bf16_round(_rand(rng, (M, N)))
    A, B, R = bf16_dev(a), bf16_dev(b), bf16_dev(r)
    lda = M if layout == 2 else K
    ldb = K if layout == 0 else N
    f32 = torch.zeros((M, N), device="cuda", dtype=torch.float32)
    c16 = torch.zeros((M, N), device="cuda", dtype=torch.bfloat16)
    res16 = torch.zeros((M, N), device="cuda", dtype=torch.bfloat16)
    mt.gemm(layout, 1, M, N, K, A, lda, B, ldb, f32, N)
    mt.gemm(layout, 0, M, N, K, A, lda, B, ldb, c16, N)
    mt.gemm(layout, 3, M, N, K, A, lda, B, ldb, res16, N, R=R, ldr=N)
    torch.cuda.synchronize()
    acc = to_np(f32)
    assert np.array_equal(to_np(c16).view(np.uint32), oracle.bf16_round(acc).view(np.uint32))
    with_r = (r + acc).astype(np.float32)
    assert np.array_equal(to_np(res16).view(np.uint32), oracle.bf16_round(with_r).view(np.uint32))


@pytest.mark.parametrize("M,F,K", [(256, 1024, 256), (200, 96, 136), (200, 96, 128)])
def test_gemm_swiglu_forward_and_backward_epilogues(M, F, K):
    torch, mt = _torch(), _mt()
    rng = np.random.default_rng(7)
    b = oracle.bf16_round(_rand(rng, (M, K)))
    wg = oracle.bf16_round(_rand(rng, (F, K), 0.1))
    wu = oracle.bf16_round(_rand(rng, (F, K), 0.1))
    Bm, W = bf16_dev(b), bf16_dev(np.concatenate([wg, wu]))
    m = torch.zeros((M, F), device="cuda", dtype=torch.bfloat16)
    gu = torch.zeros((M, 2 * F), device="cuda", dtype=torch.bfloat16)
    mt.gemm(0, 5, M, 2 * F, K, Bm, K, W, K, m, F, C2=gu, ldc2=2 * F, F=F)
    torch.cuda.synchronize()
    gt = b.astype(np.float64) @ wg.T.astype(np.float64)
    ut = b.astype(np.float64) @ wu.T.astype(np.float64)
    assert rel_fro(to_np(gu)[:, :F], gt) < 5e-3
    assert rel_fro(to_np(gu)[:, F:], ut) < 5e-3
    assert rel_fro(to_np(m), D.silu(gt) * ut) < 1e-2
    # backward epilogue: dm = dy @ W_down (NN), fused into dgate/dup, with
    # gate/up pre-activations of its own (seeded, not the product above)
    H = K
    dy = oracle.bf16_round(_rand(rng, (M, H)))
    wd = oracle.bf16_round(_rand(rng, (H, F), 0.1))
    gu_in = oracle.bf16_round(_rand(rng, (M, 2 * F), 2.0))
    dgu = torch.zeros((M, 2 * F), device="cuda", dtype=torch.bfloat16)
    mt.gemm(1, 6, M, F, H, bf16_dev(dy), H, bf16_dev(wd), F, dgu, 2 * F, C2=dgu, ldc2=2 * F,
            G=bf16_dev(gu_in), ldg=2 * F, F=F)
    torch.cuda.synchronize()
    g_bf = gu_in[:, :F].astype(np.float64)
    u_bf = gu_in[:, F:].astype(np.float64)
    dm = dy.astype(np.float64) @ wd.astype(np.float64)
    sg = 1 / (1 + np.exp(-g_bf))
    assert rel_fro(to_np(dgu)[:, :F], dm * u_bf * sg * (1 + g_bf * (1 - sg))) < 1e-2
    assert rel_fro(to_np(dgu)[:, F:], dm * D.silu(g_bf)) < 1e-2


def test_gemm_7b_gate_up_shape_sampled_rows():
    """Gate/up projection at the 7B shape (16384 x 37888 x 3584)."""
    torch, mt = _torch(), _mt()
    M, F, K = 16384, 18944, 3584
    g = torch.Generator(device="cuda").manual_seed(3)
    A = (torch.randn((M, K), device="cuda", generator=g) ).to(torch.bfloat16)
    W = (torch.randn((2 * F, K), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    m = torch.empty((M, F), device="cuda", dtype=torch.bfloat16)
    gu = torch.empty((M, 2 * F), device="cuda", dtype=torch.bfloat16)
    mt.gemm(0, 5, M, 2 * F, K, A, K, W, K, m, F, C2=gu, ldc2=2 * F, F=F)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(M, 24, replace=False)
    a = A[rows].float().cpu().numpy().astype(np.float64)
    w = W.float().cpu().numpy().astype(np.float64)
    ref = a @ w.T
    out = gu[rows].float().cpu().numpy()
    assert rel_fro(out, ref) < 5e-3
    mref = D.silu(ref[:, :F]) * ref[:, F:]
    assert rel_fro(m[rows].float().cpu().numpy(), mref) < 1e-2


# rows wider than 8192 take the wide backward kernel (column slabs of 4096)
@pytest.mark.parametrize("rows,cols", [(256, 256), (77, 3584), (130, 7168), (5, 8),
                                       (33, 12544), (20, 16384), (19, 8200)])
def test_rmsnorm_forward_backward(rows, cols):
    torch, mt = _torch(), _mt()
    rng = np.random.default_rng(rows + cols)
    x = oracle.bf16_round(_rand(rng, (rows, cols), 2.0))
    g = oracle.bf16_round(1 + 0.1 * _rand(rng, (cols,)))
    dy = oracle.bf16_round(_rand(rng, (rows, cols)))
    res = oracle.bf16_round(_rand(rng, (rows, cols)))
    X, G, DY, RES = bf16_dev(x), bf16_dev(g), bf16_dev(dy), bf16_dev(res)
    Y = torch.empty_like(X)
    rstd = torch.empty(rows, device="cuda", dtype=torch.float32)
    mt.rmsnorm_fwd(X, G, Y, rstd, rows, cols, 1e-6)
    y_ref, r_ref = D.rms_norm(x, g, 1e-6)
    dx_ref, dg_ref = D.rms_norm_backward(dy, x, g, r_ref)
    ws = torch.empty(mt.rmsnorm_bwd_workspace(rows, cols) // 4 + 1, device="cuda", dtype=torch.float32)
    DX = torch.empty_like(X)
    DG = torch.empty(cols, device="cuda", dtype=torch.bfloat16)
    mt.rmsnorm_bwd(DY, X, G, rstd, RES, DX, DG, rows, cols, ws)
    torch.cuda.synchronize()
    np.testing.assert_allclose(rstd.cpu().numpy(), r_ref[:, 0], rtol=2e-6)
    assert rel_fro(to_np(Y), y_ref) < 5e-3
    assert rel_fro(to_np(DX), dx_ref + res) < 5e-3
    assert rel_fro(to_np(DG), dg_ref) < 5e-3


@pytest.mark.parametrize("B,T,Hq,Hkv,d", [(2, 128, 4, 2, 64), (1, 77, 28, 4, 128)])
def test_rope_table_and_rotation(B, T, Hq, Hkv, d):
    torch, mt = _torch(), _mt()
    cos_t = torch.empty((T, d // 2), device="cuda", dtype=torch.float32)
    sin_t = torch.empty_like(cos_t)
    mt.rope_table(cos_t, sin_t, T, d, 1e6)
    c_ref, s_ref = D.rope_cos_sin(T, d, 1e6, np.float32)
    torch.cuda.synchronize()
    np.testing.assert_allclose(cos_t.cpu().numpy(), c_ref, rtol=0, atol=1.2e-7)
    np.testing.assert_allclose(sin_t.cpu().numpy(), s_ref, rtol=0, atol=1.2e-7)
    rng = np.random.default_rng(T)
    ld = (Hq + 2 * Hkv) * d
    qkv = oracle.bf16_round(_rand(rng, (B * T, ld)))
    Q = bf16_dev(qkv)
    mt.rope(Q, B, T, Hq, Hkv, d, cos_t, sin_t, 0)
    torch.cuda.synchronize()
    out = to_np(Q)
    nq = (Hq + Hkv) * d
    ref = D.rope(qkv[:, :nq].reshape(B, T, Hq + Hkv, d), c_ref, s_ref).reshape(B * T, nq)
    assert rel_fro(out[:, :nq], ref) < 5e-3
    np.testing.assert_array_equal(out[:, nq:], qkv[:, nq:])
    mt.rope(Q, B, T, Hq, Hkv, d, cos_t, sin_t, 1)
    torch.cuda.synchronize()
    ref_b = D.rope_backward(out[:, :nq].reshape(B, T, Hq + Hkv, d), c_ref, s_ref).reshape(B * T, nq)
    assert rel_fro(to_np(Q)[:, :nq], ref_b) < 5e-3


@pytest.mark.parametrize("rows,V", [(37, 1024), (8, 152064)])
def test_cross_entropy_rows(rows, V):
    torch, mt = _torch(), _mt()
    rng = np.random.default_rng(V)
    logits = _rand(rng, (rows, V), 3.0)
    tgt = rng.integers(0, V, rows).astype(np.int32)
    tgt[::5] = -1
    L = torch.from_numpy(logits).cuda()
    Tg = torch.from_numpy(tgt).cuda()
    dl = torch.empty((rows, V), device="cuda", dtype=torch.bfloat16)
    lp = torch.empty(rows, device="cuda", dtype=torch.float32)
    inv_n = 1.0 / max(1, int((tgt >= 0).sum()))
    mt.ce_rows(L, Tg, dl, lp, rows, V, inv_n)
    torch.cuda.synchronize()
    l64 = logits.astype(np.float64)
    mx = l64.max(1, keepdims=True)
    lse = mx[:, 0] + np.log(np.exp(l64 - mx).sum(1))
    sm = np.exp(l64 - lse[:, None])
    ref_d = np.zeros_like(sm)
    ref_l = np.zeros(rows)
    for r in range(rows):
        if tgt[r] >= 0:
            ref_d[r] = sm[r] * inv_n
            ref_d[r, tgt[r]] -= inv_n
            ref_l[r] = lse[r] - l64[r, tgt[r]]
    np.testing.assert_allclose(lp.cpu().numpy(), ref_l, rtol=1e-5, atol=1e-5)
    assert rel_fro(to_np(dl), ref_d) < 5e-3
    assert not to_np(dl)[tgt < 0].any()


ATTN_CASES = [
    # B, T, Hq, Hkv, d
    (2, 128, 4, 2, 64),     # the small parity model
    (1, 200, 6, 2, 128),    # ragged T, group 3
    (2, 300, 10, 2, 64),    # ragged T, group 5
    (1, 1024, 28, 4, 128),  # 7B heads, group 7
    (2, 700, 6, 2, 128),    # several 256-query blocks, the last ragged; 12 (block,
                            # batch, KV group) sets: one whole XCD round and a partial one
    (3, 1, 4, 4, 128),      # single token
]


def _attn_inputs(B, T, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    qkv = oracle.bf16_round(_rand(rng, (B * T, (Hq + 2 * Hkv) * d)))
    q = qkv[:, : Hq * d].reshape(B, T, Hq, d)
    k = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(B, T, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].reshape(B, T, Hkv, d)
    return qkv, q, k, v


@pytest.mark.parametrize("B,T,Hq,Hkv,d", ATTN_CASES)
def test_attention_forward_backward(B, T, Hq, Hkv, d):
    torch, mt = _torch(), _mt()
    qkv, q, k, v = _attn_inputs(B, T, Hq, Hkv, d, T + Hq)
    QKV = bf16_dev(qkv)
    O = torch.empty((B * T, Hq * d), device="cuda", dtype=torch.bfloat16)
    LSE = torch.empty((B, Hq, T), device="cuda", dtype=torch.float32)
    mt.attn_fwd(QKV, O, LSE, B, T, Hq, Hkv, d)
    torch.cuda.synchronize()
    o_ref, lse_ref = D.causal_attention(q, k, v)
    assert rel_fro(to_np(O), o_ref.reshape(B * T, Hq * d)) < 1e-2
    np.testing.assert_allclose(LSE.cpu().numpy(), lse_ref, rtol=0, atol=2e-3)
    rng = np.random.default_rng(T)
    do = oracle.bf16_round(_rand(rng, (B * T, Hq * d)))
    DO = bf16_dev(do)
    delta = torch.empty((B, Hq, T), device="cuda", dtype=torch.float32)
    DQKV = torch.full((B * T, (Hq + 2 * Hkv) * d), float("nan"), device="cuda", dtype=torch.bfloat16)
    mt.attn_bwd(QKV, O, LSE, DO, delta, DQKV, B, T, Hq, Hkv, d)
    torch.cuda.synchronize()
    # the oracle's backward from its own forward (never from GPU outputs)
    dq, dk, dv = D.causal_attention_backward(q, k, v, o_ref, lse_ref, do.reshape(B, T, Hq, d))
    out = to_np(DQKV)
    assert np.isfinite(out).all()
    # exact dq and dk vanish at T = 1 (P = 1, dS = 0): floor the denominator
    # at a small fraction of |dO| so rounding noise is compared absolutely
    floor = 1e-2 * np.linalg.norm(do)

    def err(a, b):
        return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), floor))

    assert err(out[:, : Hq * d], dq.reshape(B * T, -1)) < 2e-2
    assert err(out[:, Hq * d:(Hq + Hkv) * d], dk.reshape(B * T, -1)) < 2e-2
    assert err(out[:, (Hq + Hkv) * d:], dv.reshape(B * T, -1)) < 2e-2


def test_attention_forward_32k_sampled_heads():
    """Long-context shape (T = 32768, 7B heads): heads 0 and 27 against the
    oracle computed on those heads alone."""
    torch, mt = _torch(), _mt()
    B, T, Hq, Hkv, d = 1, 32768, 28, 4, 128
    g = torch.Generator(device="cuda").manual_seed(5)
    QKV = torch.randn((T, (Hq + 2 * Hkv) * d), device="cuda", generator=g).to(torch.bfloat16)
    O = torch.empty((T, Hq * d), device="cuda", dtype=torch.bfloat16)
    LSE = torch.empty((1, Hq, T), device="cuda", dtype=torch.float32)
    mt.attn_fwd(QKV, O, LSE, B, T, Hq, Hkv, d)
    torch.cuda.synchronize()
    qkv = QKV.float().cpu().numpy()
    for h in (0, 27):
        gkv = h * Hkv // Hq
        q = qkv[:, h * d:(h + 1) * d].reshape(1, T, 1, d)
        k = qkv[:, (Hq + gkv) * d:(Hq + gkv + 1) * d].reshape(1, T, 1, d)
        v = qkv[:, (Hq + Hkv + gkv) * d:(Hq + Hkv + gkv + 1) * d].reshape(1, T, 1, d)
        rows = np.r_[0:64, T - 2048:T]
        # rows of a causal attention depend only on keys up to the row
        o_ref, lse_ref = D.causal_attention(q, k, v, row_block=2048)
        assert rel_fro(to_np(O)[rows, h * d:(h + 1) * d], o_ref[0, rows, 0]) < 1e-2
        np.testing.assert_allclose(LSE[0, h].cpu().numpy()[rows], lse_ref[0, 0, rows], atol=2e-3)


@pytest.mark.parametrize("layout,M,N,K,epi", [
    (1, 16384, 3584, 4608, 0), (2, 37888, 3584, 2048, 0), (0, 16384, 4608, 3584, 0),
    (2, 3584, 18944, 3000, 0), (0, 16344, 4616, 3584, 0), (0, 9000, 30000, 2048, 0),
    # direct-to-LDS path with K-major operands: NN's B, TN's A and B, ragged
    # contiguous extents (clamped columns) and the fp32 accumulate epilogue
    (1, 16380, 18936, 3584, 0), (2, 37880, 3592, 2048, 0), (2, 18944, 3584, 1024, 2),
    # two stages of 64 k (NT, TN's 256 x 256 tile): the residual epilogue of
    # the down projection with a ragged M, and TN with K % 64 == 32 (the
    # 4-stage ring instead)
    (0, 16380, 3584, 18944, 3), (2, 18944, 3584, 1056, 0)])
def test_gemm_large_tiles_sampled(layout, M, N, K, epi):
    """Shapes of the 7B layer that take the 256 x 256 tile paths (ragged K on
    TN), plus ragged extents of the direct-to-LDS kernels."""
    torch, mt = _torch(), _mt()
    g = torch.Generator(device="cuda").manual_seed(M + N)
    A = torch.randn((K, M) if layout == 2 else (M, K), device="cuda", generator=g).to(torch.bfloat16)
    B = torch.randn((N, K) if layout == 0 else (K, N), device="cuda", generator=g).to(torch.bfloat16)
    R = None
    if epi == 2:
        Cm = torch.randn((M, N), device="cuda", generator=g)
        C0 = Cm.clone()
    else:
        Cm = torch.empty((M, N), device="cuda", dtype=torch.bfloat16)
        if epi == 3:
            R = torch.randn((M, N), device="cuda", generator=g).to(torch.bfloat16)
    mt.gemm(layout, epi, M, N, K, A, M if layout == 2 else K, B, K if layout == 0 else N, Cm, N,
            R=R, ldr=N)
    torch.cuda.synchronize()
    rows = np.concatenate([np.random.default_rng(1).choice(M, 14, replace=False), [0, M - 1]])
    a = (A[:, rows].t() if layout == 2 else A[rows]).float().cpu().numpy().astype(np.float64)
    b = B.float().cpu().numpy().astype(np.float64)
    ref = a @ (b.T if layout == 0 else b)
    if epi == 2:
        ref = ref + C0[rows].cpu().numpy()
        assert rel_fro(Cm[rows].cpu().numpy(), ref) < 1e-5
    else:
        if epi == 3:
            ref = ref + R[rows].float().cpu().numpy()
        assert rel_fro(Cm[rows].float().cpu().numpy(), ref) < 5e-3
    # the last column too (clamped chunks of a ragged contiguous extent)
    assert np.isfinite(Cm[rows].float().cpu().numpy()).all()


# ------------------------------------------------- fp32 debug precision
# The fp32 kernels are plain fp32 FMA with exact exp/log: against a float64
# evaluation of the same inputs the relative error is a few fp32 ulps times
# the square root of the reduction length, far below 1e-5.
F32_TOL = 1e-5

F32_GEMM_CASES = [(0, 130, 70, 100), (1, 130, 70, 100), (2, 130, 70, 100),
                  (0, 64, 128, 16), (1, 1, 3, 1), (2, 3, 1, 5)]


def f32_dev(a):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


@pytest.mark.parametrize("layout,M,N,K", F32_GEMM_CASES)
@pytest.mark.parametrize("epi", [0, 1, 2, 3])
def test_gemm_f32_layouts_and_epilogues(layout, M, N, K, epi):
    torch, mt = _torch(), _mt()
    rng = np.random.default_rng(300 + layout * 7 + epi)
    a = _rand(rng, (K, M) if layout == 2 else (M, K))
    b = _rand(rng, (N, K) if layout == 0 else (K, N))
    af, bf = a.astype(np.float64), b.astype(np.float64)
    ref = (af.T if layout == 2 else af) @ (bf.T if layout == 0 else bf)
    r = None
    Cm = torch.zeros((M, N), device="cuda", dtype=torch.float32)
    if epi == 3:
        r = _rand(rng, (M, N))
        ref = ref + r
    if epi == 2:
        init = _rand(rng, (M, N))
        Cm.copy_(torch.from_numpy(init))
        ref = ref + init
    lda = M if layout == 2 else K
    ldb = K if layout == 0 else N
    mt.gemm_f32(layout, epi, M, N, K, f32_dev(a), lda, f32_dev(b), ldb, Cm, N,
                R=None if r is None else f32_dev(r), ldr=N)
    torch.cuda.synchronize()
    assert rel_fro(Cm.cpu().numpy(), ref) < F32_TOL


@pytest.mark.parametrize("M,F,K", [(130, 96, 72), (64, 64, 64)])
def test_gemm_f32_swiglu_epilogues(M, F, K):
    torch, mt = _torch(), _mt()
    rng = np.random.default_rng(8)
    b = _rand(rng, (M, K))
    wg, wu = _rand(rng, (F, K), 0.2), _rand(rng, (F, K), 0.2)
    m = torch.zeros((M, F), device="cuda", dtype=torch.float32)
    gu = torch.zeros((M, 2 * F), device="cuda", dtype=torch.float32)
    mt.gemm_f32(0, 5, M, 2 * F, K, f32_dev(b), K, f32_dev(np.concatenate([wg, wu])), K, m, F,
                C2=gu, ldc2=2 * F, F=F)
    m4 = torch.zeros_like(m)
    mt.gemm_f32(0, 4, M, 2 * F, K, f32_dev(b), K, f32_dev(np.concatenate([wg, wu])), K, m4, F,
                F=F)
    torch.cuda.synchronize()
    gt = b.astype(np.float64) @ wg.T.astype(np.float64)
    ut = b.astype(np.float64) @ wu.T.astype(np.float64)
    assert rel_fro(gu.cpu().numpy()[:, :F], gt) < F32_TOL
    assert rel_fro(gu.cpu().numpy()[:, F:], ut) < F32_TOL
    assert rel_fro(m.cpu().numpy(), D.silu(gt) * ut) < F32_TOL
    np.testing.assert_array_equal(m4.cpu().numpy(), m.cpu().numpy())
    H = K
    dy = _rand(rng, (M, H))
    wd = _rand(rng, (H, F), 0.2)
    gu_in = _rand(rng, (M, 2 * F), 2.0)  # seeded gate/up pre-activations
    dgu = torch.zeros((M, 2 * F), device="cuda", dtype=torch.float32)
    mt.gemm_f32(1, 6, M, F, H, f32_dev(dy), H, f32_dev(wd), F, dgu, 2 * F, C2=dgu, ldc2=2 * F,
                G=f32_dev(gu_in), ldg=2 * F, F=F)
    torch.cuda.synchronize()
    g64 = gu_in[:, :F].astype(np.float64)
    u64 = gu_in[:, F:].astype(np.float64)
    dm = dy.astype(np.float64) @ wd.astype(np.float64)
    sg = 1 / (1 + np.exp(-g64))
    assert rel_fro(dgu.cpu().numpy()[:, :F], dm * u64 * sg * (1 + g64 * (1 - sg))) < F32_TOL
    assert rel_fro(dgu.cpu().numpy()[:, F:], dm * D.silu(g64)) < F32_TOL


@pytest.mark.parametrize("B,T,Hq,Hkv,d", [(2, 128, 4, 2, 64), (1, 70, 6, 2, 128),
                                          (2, 33, 10, 2, 64), (3, 1, 4, 4, 128)])
def test_attention_f32_forward_backward(B, T, Hq, Hkv, d):
    torch, mt = _torch(), _mt()
    rng = np.random.default_rng(T + 17 * Hq)
    qkv = _rand(rng, (B * T, (Hq + 2 * Hkv) * d))
    q = qkv[:, : Hq * d].reshape(B, T, Hq, d).astype(np.float64)
    k = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(B, T, Hkv, d).astype(np.float64)
    v = qkv[:, (Hq + Hkv) * d:].reshape(B, T, Hkv, d).astype(np.float64)
    QKV = f32_dev(qkv)
    O = torch.empty((B * T, Hq * d), device="cuda", dtype=torch.float32)
    LSE = torch.empty((B, Hq, T), device="cuda", dtype=torch.float32)
    mt.attn_fwd_f32(QKV, O, LSE, B, T, Hq, Hkv, d)
    do = _rand(rng, (B * T, Hq * d))
    delta = torch.empty((B, Hq, T), device="cuda", dtype=torch.float32)
    DQKV = torch.full((B * T, (Hq + 2 * Hkv) * d), float("nan"), device="cuda")
    mt.attn_bwd_f32(QKV, O, LSE, f32_dev(do), delta, DQKV, B, T, Hq, Hkv, d)
    torch.cuda.synchronize()
    o_ref, lse_ref = D.causal_attention(q, k, v)
    assert rel_fro(O.cpu().numpy(), o_ref.reshape(B * T, -1)) < F32_TOL
    np.testing.assert_allclose(LSE.cpu().numpy(), lse_ref, rtol=0, atol=1e-5)
    dq, dk, dv = D.causal_attention_backward(q, k, v, o_ref, lse_ref,
                                             do.reshape(B, T, Hq, d).astype(np.float64))
    out = DQKV.cpu().numpy()
    floor = 1e-4 * np.linalg.norm(do)  # dq, dk vanish at T = 1

    def err(a, b):
        return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), floor))

    assert err(out[:, : Hq * d], dq.reshape(B * T, -1)) < F32_TOL
    assert err(out[:, Hq * d:(Hq + Hkv) * d], dk.reshape(B * T, -1)) < F32_TOL
    assert err(out[:, (Hq + Hkv) * d:], dv.reshape(B * T, -1)) < F32_TOL


@pytest.mark.parametrize("f32", [0, 1])
def test_nonfinite_flags(f32):
    """The engine's GPU finiteness check: clean buffers give all-zero flags;
    an Inf or a NaN anywhere (first, last, middle element) sets a flag."""
    torch, mt = _torch(), _mt()
    dt = torch.float32 if f32 else torch.bfloat16
    n = 1_000_008  # elements; bytes a multiple of 16
    flags = torch.empty(2048, dtype=torch.int32, device="cuda")  # NONFINITE_BLOCKS
    g = (torch.randn(n, device="cuda") * 1e3).to(dt)
    nbytes = n * g.element_size()
    assert mt.call("mt_op_nonfinite_flags", g.data_ptr(), nbytes, f32, flags.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert int(flags.sum()) == 0
    for pos, val in ((0, float("inf")), (n - 1, float("nan")), (n // 2 + 3, float("-inf"))):
        h = g.clone()
        h[pos] = val
        assert mt.call("mt_op_nonfinite_flags", h.data_ptr(), nbytes, f32, flags.data_ptr(),
                       None) == 0
        torch.cuda.synchronize()
        assert int(flags.sum()) == 1, (pos, val)


@pytest.mark.parametrize("layout,M,N,K,epi", [
    # 896 tiles of 256 x 256 on 256 CUs: a half-full last round, split in 2
    (1, 16384, 3584, 4608, 0), (0, 16384, 3584, 3584, 3), (0, 16384, 3584, 2048, 1),
    (1, 16380, 3576, 4608, 0),
    # 1036 tiles: 12 in the last round, split in 8 (in 4 where K is short)
    (2, 3584, 18944, 16384, 0), (2, 18944, 3584, 1024, 2)])
def test_gemm_split_tail_tiles(layout, M, N, K, epi):
    """A workspace lets the tiles of a partly filled last round be split
    along K: the result matches the unsplit product to bf16 rounding (fp32
    outputs to 1e-6), matches a float64 evaluation on rows of the split
    tiles, and is the same bits on every run."""
    torch, mt = _torch(), _mt()
    g = torch.Generator(device="cuda").manual_seed(M * 7 + N + K)
    A = torch.randn((K, M) if layout == 2 else (M, K), device="cuda", generator=g).to(torch.bfloat16)
    B = torch.randn((N, K) if layout == 0 else (K, N), device="cuda", generator=g).to(torch.bfloat16)
    lda, ldb = (M if layout == 2 else K), (K if layout == 0 else N)
    R = torch.randn((M, N), device="cuda", generator=g).to(torch.bfloat16) if epi == 3 else None
    f32 = epi in (1, 2)
    init = torch.randn((M, N), device="cuda", generator=g) if epi == 2 else None

    def run(ws):
        C = (init.clone() if init is not None else
             torch.zeros((M, N), device="cuda", dtype=torch.float32 if f32 else torch.bfloat16))
        mt.gemm(layout, epi, M, N, K, A, lda, B, ldb, C, N, R=R, ldr=N, workspace=ws)
        return C

    ws = torch.empty(mt.GEMM_SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    c_whole, c_split, c_again = run(None), run(ws), run(ws)
    torch.cuda.synchronize()
    assert torch.equal(c_split, c_again)
    a, b = c_split.float(), c_whole.float()
    if f32:
        assert float((a - b).abs().max() / b.abs().max()) < 1e-6
    else:
        # one rounding of a slightly different fp32 sum: at most one bf16 step,
        # plus the fp32 summation-order difference where the sum cancels
        slack = 1e-4 * float(b.pow(2).mean().sqrt())
        excess = float(((a - b).abs() - (b.abs() * 2.0 ** -7 + slack)).max())
        assert excess <= 0, excess
    # the split tiles are the last ones launched: rows of the last tile rows
    rows = np.concatenate([np.arange(M - 3, M), M - 1 - np.random.default_rng(2).choice(M // 4, 9, replace=False)])
    at = (A[:, rows].t() if layout == 2 else A[rows]).float().cpu().numpy().astype(np.float64)
    bt = B.float().cpu().numpy().astype(np.float64)
    ref = at @ (bt.T if layout == 0 else bt)
    if epi == 2:
        ref = ref + init[rows].cpu().numpy()
    if epi == 3:
        ref = ref + R[rows].float().cpu().numpy()
    assert rel_fro(c_split[rows].float().cpu().numpy(), ref) < (1e-5 if f32 else 5e-3)
