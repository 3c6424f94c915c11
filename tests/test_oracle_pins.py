"""Pins of the CPU oracle against things other than itself.

Finite differences in float64, library routines (torch autograd, SDPA,
torch.optim.Adam, torch bfloat16 casting), closed forms and invariants that
the method implies.  CPU only.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import decoder as D

TINY = synth.ModelShape(name="fd-tiny", n_layers=2, hidden=16, n_heads=4,
                        n_kv_heads=2, head_dim=4, ffn=32, vocab=64, batch=2,
                        seq=8, ckpt_interval=1, rope_theta=10000.0)
# group size 3 (not a power of two), head_dim 8
TINY3 = synth.ModelShape(name="fd-tiny3", n_layers=1, hidden=24, n_heads=3,
                         n_kv_heads=1, head_dim=8, ffn=40, vocab=48, batch=2,
                         seq=7, ckpt_interval=1, rope_theta=10000.0)


def _fd_params(shape, seed=3, std=0.3):
    w = synth.make_weights(shape, seed=seed, std=std, dtype=np.float64)
    rng = np.random.default_rng(seed + 100)
    for n in w:
        if n.endswith("norm"):
            w[n] = 1.0 + 0.3 * rng.standard_normal(w[n].shape)
    return w


@pytest.mark.parametrize("shape", [TINY, TINY3], ids=["gqa2", "gqa3"])
def test_finite_differences_every_tensor(shape):
    w = _fd_params(shape)
    ids = synth.make_tokens(shape, seed=5)
    loss, grads = D.loss_and_grads(w, ids, shape)
    assert abs(loss - D.forward_loss(w, ids, shape)) < 1e-12
    rng = np.random.default_rng(7)
    h = 1e-6
    for name, p in w.items():
        flat = p.reshape(-1)
        g = grads[name].reshape(-1)
        assert grads[name].shape == p.shape, name
        idx = rng.choice(flat.size, size=min(6, flat.size), replace=False)
        if name == "embed":  # include rows that some token actually uses
            used = ids.reshape(-1)[:3] * p.shape[1]
            idx = np.concatenate([idx, used + 1])
        fd = []
        for i in idx:
            old = flat[i]
            flat[i] = old + h
            lp = D.forward_loss(w, ids, shape)
            flat[i] = old - h
            lm = D.forward_loss(w, ids, shape)
            flat[i] = old
            fd.append((lp - lm) / (2 * h))
        fd = np.array(fd)
        an = g[idx]
        err = np.max(np.abs(fd - an)) / max(np.max(np.abs(an)), 1e-6)
        assert err < 1e-6, (name, err, fd, an)


def test_directional_derivative():
    shape = TINY
    w = _fd_params(shape, seed=11)
    ids = synth.make_tokens(shape, seed=12)
    _, grads = D.loss_and_grads(w, ids, shape)
    rng = np.random.default_rng(13)
    dirs = {n: rng.standard_normal(p.shape) for n, p in w.items()}
    h = 1e-6
    wp = {n: p + h * dirs[n] for n, p in w.items()}
    wm = {n: p - h * dirs[n] for n, p in w.items()}
    fd = (D.forward_loss(wp, ids, shape) - D.forward_loss(wm, ids, shape)) / (2 * h)
    an = sum(float(np.sum(grads[n] * dirs[n])) for n in w)
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def _torch_loss(tw, ids, shape):
    """The decoder written with torch ops, for autograd's backward."""
    import torch
    B, T = ids.shape
    H, Hq, Hkv, d = shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim
    tids = torch.from_numpy(ids.astype(np.int64))
    x = tw["embed"][tids]
    inv = shape.rope_theta ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None, :]
    full = torch.cat([ang, ang], dim=-1)
    cos, sin = torch.cos(full)[None, :, None, :], torch.sin(full)[None, :, None, :]

    def rot(z):
        z1, z2 = z[..., : d // 2], z[..., d // 2:]
        return z * cos + torch.cat([-z2, z1], dim=-1) * sin

    def norm(z, g):
        return z * torch.rsqrt(z.pow(2).mean(-1, keepdim=True) + shape.rms_eps) * g

    for l in range(shape.n_layers):
        p = lambda n: tw[f"layers.{l}.{n}"]  # noqa: E731
        a = norm(x, p("attn_norm"))
        q = rot((a @ p("w_q").T).view(B, T, Hq, d)).transpose(1, 2)
        k = rot((a @ p("w_k").T).view(B, T, Hkv, d)).transpose(1, 2)
        v = (a @ p("w_v").T).view(B, T, Hkv, d).transpose(1, 2)
        rep = Hq // Hkv
        k = k.repeat_interleave(rep, dim=1)
        v = v.repeat_interleave(rep, dim=1)
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
        x = x + o.transpose(1, 2).reshape(B, T, Hq * d) @ p("w_o").T
        b = norm(x, p("mlp_norm"))
        x = x + (torch.nn.functional.silu(b @ p("w_gate").T) * (b @ p("w_up").T)) @ p("w_down").T
    h = norm(x, tw["final_norm"])
    logits = h @ tw["lm_head"].T
    return torch.nn.functional.cross_entropy(
        logits[:, :-1].reshape(-1, shape.vocab), tids[:, 1:].reshape(-1))


@pytest.mark.parametrize("shape", [TINY, TINY3], ids=["gqa2", "gqa3"])
def test_against_torch_autograd_float64(shape):
    import torch
    w = _fd_params(shape, seed=21)
    ids = synth.make_tokens(shape, seed=22)
    loss, grads = D.loss_and_grads(w, ids, shape)
    tw = {n: torch.tensor(p, requires_grad=True) for n, p in w.items()}
    tl = _torch_loss(tw, ids, shape)
    tl.backward()
    assert abs(float(tl.detach()) - loss) < 1e-12
    for n in w:
        ref = tw[n].grad.numpy()
        err = np.linalg.norm(grads[n] - ref) / max(np.linalg.norm(ref), 1e-30)
        assert err < 1e-10, (n, err)


def test_initial_loss_near_log_vocab():
    # logits = h W_out^T with rms(h) = 1 and W_out ~ N(0, 0.02^2): each logit
    # has variance 0.02^2 * H, so E[loss] ~= ln V + var/2.
    s = synth.CONFIGS["tiny-2l-h256"]
    w = synth.make_weights(s)
    ids = synth.make_tokens(s)
    loss = D.forward_loss(w, ids, s)
    expect = math.log(s.vocab) + 0.5 * 0.02 ** 2 * s.hidden
    assert abs(loss - expect) < 0.1, (loss, expect)


# ------------------------------------------------------------------ attention


def _rand_qkv(B, T, Hq, Hkv, d, seed, dtype=np.float64):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hq, d)).astype(dtype)
    k = rng.standard_normal((B, T, Hkv, d)).astype(dtype)
    v = rng.standard_normal((B, T, Hkv, d)).astype(dtype)
    return q, k, v


def test_attention_single_token_returns_v():
    q, k, v = _rand_qkv(2, 1, 4, 2, 8, 1)
    o, lse = D.causal_attention(q, k, v)
    np.testing.assert_allclose(o, np.repeat(v, 2, axis=2), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[:, :, 0], np.einsum("bhd,bhd->bh", q[:, 0], np.repeat(k, 2, axis=2)[:, 0]) / np.sqrt(8))


def test_attention_zero_query_is_prefix_mean():
    q, k, v = _rand_qkv(1, 9, 3, 1, 8, 2)
    q[:] = 0
    o, _ = D.causal_attention(q, k, v)
    pref = np.cumsum(v[0, :, 0, :], axis=0) / np.arange(1, 10)[:, None]
    for h in range(3):
        np.testing.assert_allclose(o[0, :, h, :], pref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (7, 1), (10, 2)])
def test_attention_matches_sdpa_and_autograd(Hq, Hkv):
    import torch
    B, T, d = 2, 13, 8
    q, k, v = _rand_qkv(B, T, Hq, Hkv, d, 3)
    o, lse = D.causal_attention(q, k, v, row_block=5)
    tq, tk, tv = (torch.tensor(z, requires_grad=True) for z in (q, k, v))
    rep = Hq // Hkv
    to = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(1, 2), tk.transpose(1, 2).repeat_interleave(rep, 1),
        tv.transpose(1, 2).repeat_interleave(rep, 1), is_causal=True).transpose(1, 2)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-12)
    s = torch.einsum("bthd,bshd->bhts", tq, tk.repeat_interleave(rep, 2)) / math.sqrt(d)
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    tl = torch.logsumexp(s.masked_fill(~mask, -float("inf")), dim=-1)
    np.testing.assert_allclose(lse, tl.detach().numpy(), rtol=1e-12, atol=1e-12)
    do = np.random.default_rng(4).standard_normal(o.shape)
    (to * torch.tensor(do)).sum().backward()
    dq, dk, dv = D.causal_attention_backward(q, k, v, o, lse, do, row_block=4)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (7, 1)])
def test_attention_rows_match_sdpa_autograd_at_those_rows(Hq, Hkv):
    """The row-restricted forms (used where the full attention is too large
    for the CPU) against torch SDPA and its autograd: o, lse and dq at the
    chosen query rows, and dk, dv of every key at or after the first of a
    run of rows that reaches the last position (later keys see no other
    queries)."""
    import torch
    B, T, d = 2, 23, 8
    q, k, v = _rand_qkv(B, T, Hq, Hkv, d, 7)
    rep = Hq // Hkv
    tq, tk, tv = (torch.tensor(z, requires_grad=True) for z in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(1, 2), tk.transpose(1, 2).repeat_interleave(rep, 1),
        tv.transpose(1, 2).repeat_interleave(rep, 1), is_causal=True).transpose(1, 2)
    do = np.random.default_rng(8).standard_normal(q.shape)
    (to * torch.tensor(do)).sum().backward()
    s = torch.einsum("bthd,bshd->bhts", tq, tk.repeat_interleave(rep, 2)) / math.sqrt(d)
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    tl = torch.logsumexp(s.masked_fill(~mask, -float("inf")), dim=-1).detach().numpy()
    # scattered rows (forward, dq) and a suffix of rows (dk, dv)
    for rows in (np.array([0, 3, 11, 22]), np.arange(15, T)):
        o, lse = D.causal_attention_rows(q[:, rows], rows, k, v)
        np.testing.assert_allclose(o, to.detach().numpy()[:, rows], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, tl[:, :, rows], rtol=1e-12, atol=1e-12)
        dq, dk, dv = D.causal_attention_backward_rows(q[:, rows], rows, k, v, o, lse, do[:, rows])
        np.testing.assert_allclose(dq, tq.grad.numpy()[:, rows], rtol=1e-10, atol=1e-11)
        if rows[-1] == T - 1 and np.all(np.diff(rows) == 1):
            r = rows[0]
            np.testing.assert_allclose(dk[:, r:], tk.grad.numpy()[:, r:], rtol=1e-10, atol=1e-11)
            np.testing.assert_allclose(dv[:, r:], tv.grad.numpy()[:, r:], rtol=1e-10, atol=1e-11)


# ----------------------------------------------------------------------- RoPE


def test_rope_invariants():
    d, T = 16, 11
    cos, sin = D.rope_cos_sin(T, d, 1e6, np.float64)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, T, 3, d))
    y = D.rope(x, cos, sin)
    # rotation: norms kept, position 0 unchanged, adjoint is the inverse
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(y[:, 0], x[:, 0])
    np.testing.assert_allclose(D.rope_backward(y, cos, sin), x, rtol=1e-12, atol=1e-13)
    # q(t).k(s) depends only on t - s
    qv, kv = rng.standard_normal(d), rng.standard_normal(d)
    Q = D.rope(np.broadcast_to(qv, (1, T, 1, d)).copy(), cos, sin)[0, :, 0]
    K = D.rope(np.broadcast_to(kv, (1, T, 1, d)).copy(), cos, sin)[0, :, 0]
    for shift in range(1, 4):
        dots = [Q[t] @ K[t - shift] for t in range(shift, T)]
        np.testing.assert_allclose(dots, dots[0], rtol=1e-11)


def test_rope_pairing_and_angle():
    # rotate-half: unit vector e_j (j < d/2) at position t goes to
    # cos(phi) e_j + sin(phi) e_{j+d/2} with phi = t * theta^(-2j/d)
    d, T, theta = 8, 6, 1e6
    cos, sin = D.rope_cos_sin(T, d, theta, np.float64)
    for j in range(d // 2):
        x = np.zeros((1, T, 1, d))
        x[..., j] = 1
        y = D.rope(x, cos, sin)[0, :, 0]
        phi = np.arange(T) * theta ** (-2.0 * j / d)
        np.testing.assert_allclose(y[:, j], np.cos(phi), atol=1e-15)
        np.testing.assert_allclose(y[:, j + d // 2], np.sin(phi), atol=1e-15)


# -------------------------------------------------------------------- RMSNorm


def test_rmsnorm_properties():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 32)) * 3
    g = np.ones(32)
    y, _ = D.rms_norm(x, g, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1, rtol=1e-13)
    y2, _ = D.rms_norm(7.5 * x, g, 0.0)
    np.testing.assert_allclose(y2, y, rtol=1e-13)
    gg = rng.standard_normal(32)
    _, r = D.rms_norm(x, gg, 0.0)
    dx, _ = D.rms_norm_backward(rng.standard_normal(x.shape), x, gg, r)
    # scale invariance: the gradient is orthogonal to x
    np.testing.assert_allclose(np.sum(dx * x, axis=-1), 0, atol=1e-12)


# ------------------------------------------------------------------------- CE


def test_head_loss_against_torch_cross_entropy():
    import torch
    rng = np.random.default_rng(8)
    B, T, H, V = 2, 6, 12, 20
    x = rng.standard_normal((B, T, H))
    g = 1 + 0.1 * rng.standard_normal(H)
    w = rng.standard_normal((V, H)) * 0.5
    ids = rng.integers(0, V, (B, T)).astype(np.int32)
    loss, dx, dg, dw, logits = D.head_forward_backward(x, g, w, ids, 1e-6, want_logits=True)
    ref = torch.nn.functional.cross_entropy(torch.tensor(logits[:, :-1].reshape(-1, V)),
                                            torch.tensor(ids[:, 1:].reshape(-1).astype(np.int64)))
    assert abs(loss - float(ref)) < 1e-13
    # dlogits rows sum to zero => dh = dlogits W has dg/dx of known form; the
    # zero-row-sum property is visible through the head bias direction:
    # adding a constant row c to W changes no loss, so sum over V of dW = 0.
    np.testing.assert_allclose(dw.sum(axis=0), 0, atol=1e-13)


def test_causality_of_logits():
    s = TINY
    w = _fd_params(s, seed=31)
    ids = synth.make_tokens(s, seed=32)
    cos, sin = D.rope_cos_sin(s.seq, s.head_dim, s.rope_theta, np.float64)

    def logits(ids_):
        x = D.embed_forward(w["embed"], ids_)
        for l in range(s.n_layers):
            x, _ = D.layer_forward(D._lw(w, l), x, s, cos, sin)
        *_, lg = D.head_forward_backward(x, w["final_norm"], w["lm_head"], ids_, s.rms_eps, want_logits=True)
        return lg

    base = logits(ids)
    t = 4
    ids2 = ids.copy()
    ids2[:, t + 1:] = (ids2[:, t + 1:] + 7) % s.vocab
    np.testing.assert_array_equal(logits(ids2)[:, : t + 1], base[:, : t + 1])


def test_embed_backward_brute_force():
    rng = np.random.default_rng(9)
    ids = rng.integers(0, 5, (3, 7)).astype(np.int32)
    dx0 = rng.standard_normal((3, 7, 4))
    dE = D.embed_backward(dx0, ids, 6)
    ref = np.zeros((6, 4))
    for b in range(3):
        for t in range(7):
            ref[ids[b, t]] += dx0[b, t]
    np.testing.assert_array_equal(dE, ref)
    assert not dE[5].any()


# ----------------------------------------------------------------------- Adam


def test_adam_first_step_closed_form():
    rng = np.random.default_rng(10)
    p = rng.standard_normal(1000).astype(np.float64)
    g = rng.standard_normal(1000) * 1e-3
    g[:10] = 0
    p1, m1, v1 = D.adam_update(p, np.zeros_like(p), np.zeros_like(p), g, 1, 1e-4, 0.9, 0.999, 1e-8)
    np.testing.assert_allclose(p1 - p, -1e-4 * g / (np.abs(g) + 1e-8), rtol=1e-9, atol=1e-18)
    np.testing.assert_array_equal(p1[:10], p[:10])
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-14)
    np.testing.assert_allclose(v1, 0.001 * g * g, rtol=1e-13)


def test_adam_constant_gradient_same_update_each_step():
    g = np.array([0.3, -2.0, 1e-3])
    p = np.zeros(3)
    m = np.zeros(3)
    v = np.zeros(3)
    deltas = []
    for t in range(1, 6):
        p2, m, v = D.adam_update(p, m, v, g, t, 1e-3, 0.9, 0.999, 0.0)
        deltas.append(p2 - p)
        p = p2
    for dlt in deltas:
        np.testing.assert_allclose(dlt, -1e-3 * np.sign(g), rtol=1e-12)


def test_adam_matches_torch_optim_adam():
    import torch
    rng = np.random.default_rng(11)
    p0 = rng.standard_normal(257)
    gs = [rng.standard_normal(257) for _ in range(4)]
    tp = torch.nn.Parameter(torch.tensor(p0))
    opt = torch.optim.Adam([tp], lr=1e-3, betas=(0.9, 0.999), eps=1e-8)
    p, m, v = p0.copy(), np.zeros(257), np.zeros(257)
    for t, g in enumerate(gs, start=1):
        tp.grad = torch.tensor(g)
        opt.step()
        p, m, v = D.adam_update(p, m, v, g, t, 1e-3, 0.9, 0.999, 1e-8)
    np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)


def test_step_lowers_loss_to_first_order():
    s = TINY
    w = _fd_params(s, seed=41, std=0.1)
    ids = synth.make_tokens(s, seed=42)
    s2 = s.with_(lr=1e-5)
    loss, grads, newp, _ = D.train_step(w, ids, s2)
    new_loss = D.forward_loss(newp, ids, s)
    pred = -1e-5 * sum(float(np.sum(np.abs(g) / (np.abs(g) + 1e-8) * np.abs(g))) for g in grads.values())
    assert new_loss < loss
    assert abs((new_loss - loss) - pred) < 0.05 * abs(pred), (new_loss - loss, pred)


# ------------------------------------------------------- schedule invariance


@pytest.mark.parametrize("K", [1, 2, 3, 5])
def test_streamed_equals_resident_bitwise(K):
    s = TINY.with_(n_layers=5)
    w = synth.make_weights(s, seed=51, std=0.2, dtype=np.float32)
    ids = synth.make_tokens(s, seed=52)
    l1, g1 = D.loss_and_grads(w, ids, s, mode="resident")
    l2, g2 = D.loss_and_grads(w, ids, s, mode="streamed", ckpt_interval=K)
    assert l1 == l2
    for n in g1:
        np.testing.assert_array_equal(g1[n], g2[n], err_msg=n)


# ---------------------------------------------------------------- bfloat16


def test_bf16_rne_against_torch_cast():
    import torch
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x00000001,
                        0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F80C000, 0x7F7F8000,
                        0x00008000, 0x00018000], dtype=np.uint32)
    bits = np.concatenate([bits, special])
    x = bits.view(np.float32)
    mine = D.bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert np.all((mine[nan] & 0x7FFF) > 0x7F80)


# --------------------------------------------------- architecture vs Table 5


def _golden(name):
    import os
    p = os.path.join(os.path.dirname(__file__), "golden", name)
    rows = []
    for line in open(p):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


def test_param_shapes_reproduce_table5():
    base = synth.CONFIGS["qwen2.5-7b-b16-t1024"]
    for layers, billions in _golden("table5_depth.txt"):
        s = base.with_(n_layers=int(layers))
        n = sum(int(np.prod(v)) for v in synth.param_shapes(s).values())
        assert round(n / 1e9, 2) == float(billions), (layers, n)
    # the alternatives the reading rules out: tied head, full-width K/V
    s = base
    n = sum(int(np.prod(v)) for v in synth.param_shapes(s).values())
    assert round((n - s.vocab * s.hidden) / 1e9, 2) != 7.62
    assert round((n + 2 * s.n_layers * s.hidden * (s.q_dim - s.kv_dim)) / 1e9, 2) != 7.62
