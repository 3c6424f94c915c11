"""Parity at the sizes the product runs, through the C ABI, against the
oracle: the 7B-wide LM head at its full vocabulary with more than 2^31 fp32
logits, the attention backward over a 32K-token sequence (one whole KV
group), and the attention at 512K tokens, where the fused QKV activation
and its gradient pass 2^31 elements (sampled query rows and the last key
block, which only the last rows' queries see).

Each test prints its phases as they end, past pytest's output capture (the
oracle runs for up to a minute or more on the host cores)."""
import sys
import time

import numpy as np
import pytest

import oracle
import synth
from oracle import decoder as D

pytestmark = pytest.mark.gpu

LOSS_TOL = 1e-2
REL_TOL = 2e-2


@pytest.fixture
def say(capsys):
    def _say(msg):
        with capsys.disabled():
            print(f"[{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)
    return _say


def _env():
    import torch
    from layer_streamed_amd import mt
    assert torch.cuda.is_available()
    return torch, mt


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-30))


@pytest.mark.timeout(1200)
def test_full_vocab_step_7b_width_past_2_31_logits(say):
    """One streamed step of a one-layer model at the 7B width and vocabulary
    (H 3584, 28/4 heads, F 18944, V 152064) on 14 x 1024 tokens: the LM
    head runs all 14336 tokens as one chunk, 14336 x 152064 = 2.18e9 fp32
    logits (past 2^31 elements), through the fp32-epilogue logits GEMM, the
    cross-entropy rows and the NN / TN head GEMMs with K = V.  Loss, every
    gradient and every updated master against the oracle's train_step."""
    torch, mt = _env()
    s = synth.CONFIGS["qwen2.5-7b-b16-t1024"].with_(n_layers=1, batch=14, seq=1024,
                                                     ckpt_interval=1)
    assert s.tokens * s.vocab > 2 ** 31
    say(f"full-vocab step: drawing weights ({s.tokens} tokens, V {s.vocab})")
    w = synth.make_weights(s, seed=31, bf16_exact=True)
    ids = synth.make_tokens(s, seed=32)
    m = mt.Model(s, keep_grads=1)
    try:
        m.set_params(w)
        arena = torch.empty(m.arena_bytes(s.batch, s.seq), dtype=torch.uint8, device="cuda")
        streams = [torch.cuda.Stream() for _ in range(3)]
        loss_gpu, _ = m.step(ids, arena, streams)
        del arena
        names = synth.param_names(s)
        g_grad = {n: m.get(n, mt.GET_GRAD) for n in names}
        g_master = {n: m.get(n, mt.GET_MASTER) for n in names}
    finally:
        m.close()
    say(f"full-vocab step: GPU loss {loss_gpu:.5f}; oracle train_step running")
    loss, grads, newp, _ = D.train_step(w, ids, s)
    say(f"full-vocab step: oracle loss {loss:.5f}")
    assert abs(loss_gpu - loss) < LOSS_TOL, (loss_gpu, loss)
    for n in names:
        eg, ep = rel(g_grad[n], grads[n]), rel(g_master[n], newp[n])
        say(f"  {n}: grad {eg:.2e}, master {ep:.2e}")
        assert eg < REL_TOL, (n, eg)
        assert ep < REL_TOL, (n, ep)


def _qkv_cols(Hq, Hkv, d, h=None, kv=None, which="q"):
    if which == "q":
        return slice(h * d, (h + 1) * d)
    if which == "k":
        return slice((Hq + kv) * d, (Hq + kv + 1) * d)
    return slice((Hq + Hkv + kv) * d, (Hq + Hkv + kv + 1) * d)


@pytest.mark.timeout(900)
def test_attention_32k_backward_one_kv_group(say):
    """T = 32768 with the 7B heads (28 query / 4 KV heads, d 128): forward
    and the full backward on the GPU; the oracle computes KV group 0 (query
    heads 0-6, which share KV head 0) entirely: o and lse of those heads,
    dq of those heads at every position, dk and dv of KV head 0 at every
    key (256 key blocks, each summing 7 heads over up to 256 query blocks,
    launched in the kernel's most-query-tiles-first order)."""
    torch, mt = _env()
    B, T, Hq, Hkv, d = 1, 32768, 28, 4, 128
    rng = np.random.default_rng(41)
    qkv = oracle.bf16_round(rng.standard_normal((T, (Hq + 2 * Hkv) * d)).astype(np.float32))
    do = oracle.bf16_round(rng.standard_normal((T, Hq * d)).astype(np.float32))
    QKV = torch.from_numpy(qkv).cuda().to(torch.bfloat16)
    DO = torch.from_numpy(do).cuda().to(torch.bfloat16)
    O = torch.empty((T, Hq * d), device="cuda", dtype=torch.bfloat16)
    LSE = torch.empty((1, Hq, T), device="cuda", dtype=torch.float32)
    delta = torch.empty((1, Hq, T), device="cuda", dtype=torch.float32)
    DQKV = torch.full((T, (Hq + 2 * Hkv) * d), float("nan"), device="cuda", dtype=torch.bfloat16)
    mt.attn_fwd(QKV, O, LSE, B, T, Hq, Hkv, d)
    mt.attn_bwd(QKV, O, LSE, DO, delta, DQKV, B, T, Hq, Hkv, d)
    torch.cuda.synchronize()
    o_gpu = O[:, : 7 * d].float().cpu().numpy().reshape(T, 7, d)
    lse_gpu = LSE[0, :7].cpu().numpy()
    dqkv = DQKV.float().cpu().numpy()
    del QKV, DO, O, LSE, delta, DQKV
    say("attention 32K: GPU done; oracle forward for query heads 0-6")
    q = qkv[:, : 7 * d].reshape(1, T, 7, d)
    k = qkv[:, _qkv_cols(Hq, Hkv, d, kv=0, which="k")].reshape(1, T, 1, d)
    v = qkv[:, _qkv_cols(Hq, Hkv, d, kv=0, which="v")].reshape(1, T, 1, d)
    dor = do[:, : 7 * d].reshape(1, T, 7, d)
    o_ref, lse_ref = D.causal_attention(q, k, v, row_block=2048)
    say("attention 32K: oracle backward")
    dq, dk, dv = D.causal_attention_backward(q, k, v, o_ref, lse_ref, dor, row_block=2048)
    say("attention 32K: comparing")
    for h in range(7):
        assert rel(o_gpu[:, h], o_ref[0, :, h]) < 1e-2, h
        np.testing.assert_allclose(lse_gpu[h], lse_ref[0, h], rtol=0, atol=2e-3)
        assert rel(dqkv[:, h * d:(h + 1) * d], dq[0, :, h]) < REL_TOL, h
    assert rel(dqkv[:, _qkv_cols(Hq, Hkv, d, kv=0, which="k")], dk[0, :, 0]) < REL_TOL
    assert rel(dqkv[:, _qkv_cols(Hq, Hkv, d, kv=0, which="v")], dv[0, :, 0]) < REL_TOL
    assert np.isfinite(dqkv).all()


@pytest.mark.timeout(900)
def test_attention_512k_sampled_rows_and_last_key_block(say):
    """T = 524288 with the 7B heads: the fused QKV activation and its
    gradient hold 524288 x 4608 = 2.4e9 elements, past 2^31, so every row
    past 466033 is addressed beyond 32-bit offsets.  Inputs from a seeded
    generator on the device; the oracle takes, for KV groups 0 and 3
    (query heads 0-6 and 21-27), the first 64 query rows, the 64 rows
    around the 2^31-element boundary and the last 128 rows: o, lse and dq
    at those rows (each row's softmax over all its keys), and dk, dv of the
    last key block (128 keys, whose only queries are the last 128 rows)."""
    torch, mt = _env()
    B, T, Hq, Hkv, d = 1, 524288, 28, 4, 128
    ld = (Hq + 2 * Hkv) * d
    assert (T - 1) * ld > 2 ** 31
    g = torch.Generator(device="cuda").manual_seed(43)
    QKV = torch.randn((T, ld), device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)
    DO = torch.randn((T, Hq * d), device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)
    O = torch.empty((T, Hq * d), device="cuda", dtype=torch.bfloat16)
    LSE = torch.empty((1, Hq, T), device="cuda", dtype=torch.float32)
    delta = torch.empty((1, Hq, T), device="cuda", dtype=torch.float32)
    DQKV = torch.full((T, ld), float("nan"), device="cuda", dtype=torch.bfloat16)
    say("attention 512K: forward")
    mt.attn_fwd(QKV, O, LSE, B, T, Hq, Hkv, d)
    torch.cuda.synchronize()
    say("attention 512K: backward")
    mt.attn_bwd(QKV, O, LSE, DO, delta, DQKV, B, T, Hq, Hkv, d)
    torch.cuda.synchronize()
    cross = (2 ** 31) // ld  # last row whose start offset is below 2^31
    rows = np.r_[0:64, cross - 31:cross + 33, T - 128:T]
    rows_t = torch.from_numpy(rows).cuda()
    say("attention 512K: GPU done; oracle on sampled rows")
    for kv in (0, 3):
        heads = list(range(kv * 7, kv * 7 + 7))
        k = QKV[:, _qkv_cols(Hq, Hkv, d, kv=kv, which="k")].float().cpu().numpy()
        v = QKV[:, _qkv_cols(Hq, Hkv, d, kv=kv, which="v")].float().cpu().numpy()
        qr = QKV[rows_t, heads[0] * d:(heads[-1] + 1) * d].float().cpu().numpy()
        dor = DO[rows_t, heads[0] * d:(heads[-1] + 1) * d].float().cpu().numpy()
        n = len(rows)
        o_ref, lse_ref = D.causal_attention_rows(qr.reshape(1, n, 7, d), rows,
                                                 k.reshape(1, T, 1, d), v.reshape(1, T, 1, d))
        dq, dk, dv = D.causal_attention_backward_rows(
            qr.reshape(1, n, 7, d), rows, k.reshape(1, T, 1, d), v.reshape(1, T, 1, d),
            o_ref, lse_ref, dor.reshape(1, n, 7, d))
        o_gpu = O[rows_t, heads[0] * d:(heads[-1] + 1) * d].float().cpu().numpy().reshape(n, 7, d)
        lse_gpu = LSE[0, heads[0]:heads[-1] + 1][:, rows_t].cpu().numpy()
        dq_gpu = DQKV[rows_t, heads[0] * d:(heads[-1] + 1) * d].float().cpu().numpy()
        for j in range(7):
            assert rel(o_gpu[:, j], o_ref[0, :, j]) < 1e-2, (kv, j)
            np.testing.assert_allclose(lse_gpu[j], lse_ref[0, j], rtol=0, atol=2e-3)
            assert rel(dq_gpu.reshape(n, 7, d)[:, j], dq[0, :, j]) < REL_TOL, (kv, j)
        last = slice(T - 128, T)
        dk_gpu = DQKV[last, _qkv_cols(Hq, Hkv, d, kv=kv, which="k")].float().cpu().numpy()
        dv_gpu = DQKV[last, _qkv_cols(Hq, Hkv, d, kv=kv, which="v")].float().cpu().numpy()
        assert rel(dk_gpu, dk[0, last, 0]) < REL_TOL, kv
        assert rel(dv_gpu, dv[0, last, 0]) < REL_TOL, kv
        assert np.isfinite(dq_gpu).all() and np.isfinite(dk_gpu).all()
        say(f"attention 512K: KV group {kv} matches")
