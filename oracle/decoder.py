"""Plain NumPy decoder forward, backward and CPU Adam step (test oracle).

What is computed: one full-batch training step of a pre-norm GQA decoder
(Qwen2.5 shape, MegaTrain page, Table 2) whose parameters and Adam states are
held on the host and whose optimizer step runs on the CPU (MegaTrain
Abstract; blog summary section 1).  Streaming, double buffering and the
stateless template (blog summary sections 2 and 4) change where the work
runs, not what it computes, so this oracle is the plain definition written
out, plus the segmented checkpoint-and-recompute schedule (blog summary
section 3) as a second mode that must give bitwise the same result.

Readings where the pages are silent (each is listed in the design notes):
pre-norm residual blocks with no biases and untied head; RMSNorm in the
activation dtype with gains starting at 1; rotate-half RoPE with angles in
float64; contiguous GQA grouping; causal softmax scaled by 1/sqrt(d);
next-token loss averaged over B*(T-1) positions; PyTorch-style Adam.

Layout: activations [B, T, features]; weights [out, in] so that a linear
layer is ``x @ W.T``.  Parameter names follow ``synth.param_names``.

Test infrastructure only: nothing in the product may import this module.
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------
# RMSNorm
# --------------------------------------------------------------------------


def rms_norm(x, gain, eps):
    """y = x / sqrt(mean(x^2) + eps) * gain over the last axis.

    Returns (y, rstd) with rstd = 1/sqrt(mean(x^2)+eps) kept for backward.
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(ms + x.dtype.type(eps))
    return x * rstd * gain, rstd


def rms_norm_backward(dy, x, gain, rstd):
    """Gradient of rms_norm.  With xh = x*rstd and e = dy*gain:
    dx = rstd * (e - xh * mean(e*xh)),  dgain = sum over rows of dy*xh."""
    xh = x * rstd
    dgain = np.sum((dy * xh).reshape(-1, x.shape[-1]), axis=0)
    e = dy * gain
    dx = rstd * (e - xh * np.mean(e * xh, axis=-1, keepdims=True))
    return dx, dgain


# --------------------------------------------------------------------------
# Rotary position embedding (rotate-half pairing (j, j + d/2))
# --------------------------------------------------------------------------


def rope_cos_sin(seq, head_dim, theta, dtype=np.float32):
    """cos/sin tables [seq, head_dim/2]: angle(t, j) = t * theta^(-2j/d).

    Angles are formed in float64 and the tables stored in ``dtype``.
    """
    half = head_dim // 2
    j = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / head_dim)
    ang = np.arange(seq, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x, cos, sin):
    """Rotate each pair (x_j, x_{j+d/2}) of x [B, T, heads, d] by angle(t, j)."""
    half = x.shape[-1] // 2
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_backward(dy, cos, sin):
    """Adjoint of rope: rotation by the negative angle."""
    half = dy.shape[-1] // 2
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    d1, d2 = dy[..., :half], dy[..., half:]
    return np.concatenate([d1 * c + d2 * s, d2 * c - d1 * s], axis=-1)


# --------------------------------------------------------------------------
# Causal grouped-query attention
# --------------------------------------------------------------------------


def _kv_head(h, n_heads, n_kv_heads):
    """Contiguous grouping: query head h reads key/value head h*Hkv//Hq."""
    return (h * n_kv_heads) // n_heads


def causal_attention(q, k, v, row_block=None):
    """o = softmax(q k^T / sqrt(d), causal) v per query head.

    q [B, T, Hq, d]; k, v [B, T, Hkv, d].  Returns o [B, T, Hq, d] and the
    row log-sum-exp lse [B, Hq, T] of the scaled, masked scores.  Each row's
    softmax is exact; ``row_block`` only bounds the score block held at once.
    """
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    scale = q.dtype.type(1.0 / math.sqrt(d))
    rb = T if row_block is None else row_block
    o = np.empty_like(q)
    lse = np.empty((B, Hq, T), dtype=q.dtype)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            kk, vv = k[b, :, g, :], v[b, :, g, :]
            for r0 in range(0, T, rb):
                r1 = min(T, r0 + rb)
                s = (q[b, r0:r1, h, :] @ kk[:r1].T) * scale
                t_idx = np.arange(r0, r1)[:, None]
                s_idx = np.arange(r1)[None, :]
                s = np.where(s_idx <= t_idx, s, -np.inf)
                mx = np.max(s, axis=-1, keepdims=True)
                p = np.exp(s - mx)
                den = np.sum(p, axis=-1, keepdims=True)
                o[b, r0:r1, h, :] = (p / den) @ vv[:r1]
                lse[b, h, r0:r1] = (mx + np.log(den))[:, 0]
    return o, lse


def causal_attention_backward(q, k, v, o, lse, do, row_block=None):
    """Gradients of causal_attention.  With P = exp(S - lse):
    dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
    dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d); dK and dV are summed over
    the query heads that share a key/value head."""
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    scale = q.dtype.type(1.0 / math.sqrt(d))
    rb = T if row_block is None else row_block
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            kk, vv = k[b, :, g, :], v[b, :, g, :]
            for r0 in range(0, T, rb):
                r1 = min(T, r0 + rb)
                qq = q[b, r0:r1, h, :]
                dd = do[b, r0:r1, h, :]
                s = (qq @ kk[:r1].T) * scale
                t_idx = np.arange(r0, r1)[:, None]
                s_idx = np.arange(r1)[None, :]
                p = np.where(s_idx <= t_idx, np.exp(s - lse[b, h, r0:r1][:, None]), 0)
                p = p.astype(q.dtype)
                delta = np.sum(dd * o[b, r0:r1, h, :], axis=-1, keepdims=True)
                dv[b, :r1, g, :] += p.T @ dd
                dp = dd @ vv[:r1].T
                ds = p * (dp - delta)
                dq[b, r0:r1, h, :] = (ds @ kk[:r1]) * scale
                dk[b, :r1, g, :] += (ds.T @ qq) * scale
    return dq, dk, dv


def causal_attention_rows(q_rows, rows, k, v):
    """causal_attention at the query positions ``rows`` only.

    q_rows [B, n, Hq, d] are the queries at positions rows[0..n) (ints,
    each in [0, T)); k, v [B, T, Hkv, d].  Query position t attends to keys
    0..t with the exact softmax, as in causal_attention; the result is that
    function's o and lse at those positions: o [B, n, Hq, d], lse [B, Hq, n].
    """
    B, n, Hq, d = q_rows.shape
    Hkv = k.shape[2]
    rows = np.asarray(rows)
    scale = q_rows.dtype.type(1.0 / math.sqrt(d))
    r1 = int(rows.max()) + 1
    o = np.empty_like(q_rows)
    lse = np.empty((B, Hq, n), dtype=q_rows.dtype)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            s = (q_rows[b, :, h, :] @ k[b, :r1, g, :].T) * scale
            s = np.where(np.arange(r1)[None, :] <= rows[:, None], s, -np.inf)
            mx = np.max(s, axis=-1, keepdims=True)
            p = np.exp(s - mx)
            den = np.sum(p, axis=-1, keepdims=True)
            o[b, :, h, :] = (p / den) @ v[b, :r1, g, :]
            lse[b, h, :] = (mx + np.log(den))[:, 0]
    return o, lse


def causal_attention_backward_rows(q_rows, rows, k, v, o_rows, lse_rows, do_rows):
    """causal_attention_backward restricted to the query positions ``rows``
    (layouts as in causal_attention_rows; o_rows, lse_rows, do_rows at those
    positions).  Returns dq at those positions and the part of dk, dv
    [B, T, Hkv, d] that those queries contribute.  Key s receives
    contributions only from queries t >= s, so when ``rows`` holds every
    position from some r on, dk and dv are complete for the keys s >= r."""
    B, n, Hq, d = q_rows.shape
    T, Hkv = k.shape[1], k.shape[2]
    rows = np.asarray(rows)
    scale = q_rows.dtype.type(1.0 / math.sqrt(d))
    r1 = int(rows.max()) + 1
    dq = np.zeros_like(q_rows)
    dk = np.zeros((B, T, Hkv, d), dtype=k.dtype)
    dv = np.zeros((B, T, Hkv, d), dtype=v.dtype)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            kk, vv = k[b, :r1, g, :], v[b, :r1, g, :]
            qq, dd = q_rows[b, :, h, :], do_rows[b, :, h, :]
            s = (qq @ kk.T) * scale
            mask = np.arange(r1)[None, :] <= rows[:, None]
            p = np.where(mask, np.exp(s - lse_rows[b, h, :][:, None]), 0).astype(q_rows.dtype)
            delta = np.sum(dd * o_rows[b, :, h, :], axis=-1, keepdims=True)
            dv[b, :r1, g, :] += p.T @ dd
            ds = p * (dd @ vv.T - delta)
            dq[b, :, h, :] = (ds @ kk) * scale
            dk[b, :r1, g, :] += (ds.T @ qq) * scale
    return dq, dk, dv


# --------------------------------------------------------------------------
# SwiGLU
# --------------------------------------------------------------------------


def silu(z):
    return z / (1 + np.exp(-z))


def _sigmoid(z):
    return 1 / (1 + np.exp(-z))


# --------------------------------------------------------------------------
# One decoder layer (the stateless template's computation)
# --------------------------------------------------------------------------


def _lw(params, layer):
    p = f"layers.{layer}."
    return {k: params[p + k] for k in ("attn_norm", "w_q", "w_k", "w_v", "w_o",
                                        "mlp_norm", "w_gate", "w_up", "w_down")}


def layer_forward(w, x, shape, cos, sin):
    """x_out = layer(x) with its internals kept for backward.

    a = rms(x)*g1; q,k,v = a W^T; rope(q,k); o = attn(q,k,v);
    x_mid = x + o Wo^T; b = rms(x_mid)*g2; m = silu(b Wg^T) * (b Wu^T);
    x_out = x_mid + m Wd^T.
    """
    B, T, H = x.shape
    Hq, Hkv, d = shape.n_heads, shape.n_kv_heads, shape.head_dim
    a, r1 = rms_norm(x, w["attn_norm"], shape.rms_eps)
    q = (a @ w["w_q"].T).reshape(B, T, Hq, d)
    k = (a @ w["w_k"].T).reshape(B, T, Hkv, d)
    v = (a @ w["w_v"].T).reshape(B, T, Hkv, d)
    q = rope(q, cos, sin)
    k = rope(k, cos, sin)
    o, lse = causal_attention(q, k, v)
    o = o.reshape(B, T, Hq * d)
    x_mid = x + o @ w["w_o"].T
    b, r2 = rms_norm(x_mid, w["mlp_norm"], shape.rms_eps)
    gt = b @ w["w_gate"].T
    u = b @ w["w_up"].T
    m = silu(gt) * u
    x_out = x_mid + m @ w["w_down"].T
    saved = dict(x=x, a=a, r1=r1, q=q, k=k, v=v, o=o, lse=lse, x_mid=x_mid,
                 b=b, r2=r2, gt=gt, u=u, m=m)
    return x_out, saved


def _wgrad(dy, x):
    """dW = dy^T x with the token axes (B, T) flattened: [out, in]."""
    return dy.reshape(-1, dy.shape[-1]).T @ x.reshape(-1, x.shape[-1])


def layer_backward(w, saved, dy, shape, cos, sin):
    """Backward through layer_forward given dL/dx_out; returns (dx, grads)."""
    B, T, H = dy.shape
    Hq, Hkv, d = shape.n_heads, shape.n_kv_heads, shape.head_dim
    s = saved
    g = {}
    # down projection
    dm = dy @ w["w_down"]
    g["w_down"] = _wgrad(dy, s["m"])
    # SwiGLU: m = silu(gt) * u
    sg = _sigmoid(s["gt"])
    dgt = dm * s["u"] * (sg * (1 + s["gt"] * (1 - sg)))
    du = dm * silu(s["gt"])
    db = dgt @ w["w_gate"] + du @ w["w_up"]
    g["w_gate"] = _wgrad(dgt, s["b"])
    g["w_up"] = _wgrad(du, s["b"])
    # second norm and residual
    dxm_n, g["mlp_norm"] = rms_norm_backward(db, s["x_mid"], w["mlp_norm"], s["r2"])
    dx_mid = dy + dxm_n
    # output projection
    do = dx_mid @ w["w_o"]
    g["w_o"] = _wgrad(dx_mid, s["o"])
    # attention
    dq, dk, dv = causal_attention_backward(
        s["q"], s["k"], s["v"], s["o"].reshape(B, T, Hq, d), s["lse"],
        do.reshape(B, T, Hq, d))
    dq = rope_backward(dq, cos, sin).reshape(B, T, Hq * d)
    dk = rope_backward(dk, cos, sin).reshape(B, T, Hkv * d)
    dv = dv.reshape(B, T, Hkv * d)
    da = dq @ w["w_q"] + dk @ w["w_k"] + dv @ w["w_v"]
    g["w_q"] = _wgrad(dq, s["a"])
    g["w_k"] = _wgrad(dk, s["a"])
    g["w_v"] = _wgrad(dv, s["a"])
    # first norm and residual
    dx_n, g["attn_norm"] = rms_norm_backward(da, s["x"], w["attn_norm"], s["r1"])
    dx = dx_mid + dx_n
    return dx, g


# --------------------------------------------------------------------------
# Embedding, head and loss
# --------------------------------------------------------------------------


def embed_forward(E, ids):
    """x0[b, t] = E[ids[b, t]]."""
    return E[ids]


def embed_backward(dx0, ids, vocab):
    """dE[v] = sum of dx0[b, t] over positions with ids[b, t] = v, summed
    in token order (row-major over [B, T])."""
    dE = np.zeros((vocab, dx0.shape[-1]), dtype=dx0.dtype)
    np.add.at(dE, ids.reshape(-1), dx0.reshape(-1, dx0.shape[-1]))
    return dE


def head_forward_backward(x, gain, w_out, ids, eps, want_logits=False):
    """Final norm, LM head and next-token cross-entropy, forward and backward.

    h = rms(x)*g_f; logits = h W_out^T; loss = mean over b and t < T-1 of
    logsumexp(logits[b,t]) - logits[b, t, ids[b, t+1]].  The last position
    of every sequence has no target and gets zero gradient.
    Returns loss, dx, dg_f, dW_out (and logits if asked).
    """
    B, T, H = x.shape
    h, rf = rms_norm(x, gain, eps)
    logits = h @ w_out.T
    lg = logits[:, :-1, :]
    tgt = ids[:, 1:]
    mx = np.max(lg, axis=-1, keepdims=True)
    ex = np.exp(lg - mx)
    den = np.sum(ex, axis=-1, keepdims=True)
    lse = mx + np.log(den)
    picked = np.take_along_axis(lg, tgt[..., None], axis=-1)
    n_tgt = B * (T - 1)
    loss = np.sum(lse - picked) / n_tgt
    dlogits = np.zeros_like(logits)
    sm = ex / den
    onehot = np.zeros_like(sm)
    np.put_along_axis(onehot, tgt[..., None], 1, axis=-1)
    dlogits[:, :-1, :] = (sm - onehot) / lg.dtype.type(n_tgt)
    dh = dlogits @ w_out
    dw_out = _wgrad(dlogits, h)
    dx, dgf = rms_norm_backward(dh, x, gain, rf)
    out = (loss, dx, dgf, dw_out)
    if want_logits:
        out = out + (logits,)
    return out


# --------------------------------------------------------------------------
# Whole step: resident and streamed (checkpoint + recompute) schedules
# --------------------------------------------------------------------------


def forward_loss(params, ids, shape):
    """Loss only (used by finite-difference pins)."""
    T = ids.shape[1]
    dt = params["embed"].dtype
    cos, sin = rope_cos_sin(T, shape.head_dim, shape.rope_theta, dt)
    x = embed_forward(params["embed"], ids)
    for l in range(shape.n_layers):
        x, _ = layer_forward(_lw(params, l), x, shape, cos, sin)
    loss, *_ = head_forward_backward(x, params["final_norm"], params["lm_head"],
                                     ids, shape.rms_eps)
    return loss


def loss_and_grads(params, ids, shape, mode="resident", ckpt_interval=None):
    """Loss and the gradient of every parameter.

    mode="resident": the forward keeps every layer's internals.
    mode="streamed": the forward keeps only the inputs of layers l with
    l % K == 0; the backward walks segments from the last, re-runs the
    segment's forward from its checkpoint to rebuild each layer input, and
    recomputes each layer's internals just before its backward.
    """
    L = shape.n_layers
    T = ids.shape[1]
    dt = params["embed"].dtype
    cos, sin = rope_cos_sin(T, shape.head_dim, shape.rope_theta, dt)
    K = shape.ckpt_interval if ckpt_interval is None else ckpt_interval
    grads = {}
    x = embed_forward(params["embed"], ids)
    saved_all, ckpts = [], {}
    for l in range(L):
        if mode == "streamed" and l % K == 0:
            ckpts[l] = x
        x, saved = layer_forward(_lw(params, l), x, shape, cos, sin)
        if mode == "resident":
            saved_all.append(saved)
    loss, dx, grads["final_norm"], grads["lm_head"] = head_forward_backward(
        x, params["final_norm"], params["lm_head"], ids, shape.rms_eps)
    if mode == "resident":
        for l in reversed(range(L)):
            dx, g = layer_backward(_lw(params, l), saved_all[l], dx, shape, cos, sin)
            for k2, val in g.items():
                grads[f"layers.{l}.{k2}"] = val
    elif mode == "streamed":
        for start in reversed(range(0, L, K)):
            end = min(start + K, L)
            inputs = [ckpts[start]]
            for l in range(start, end - 1):
                y, _ = layer_forward(_lw(params, l), inputs[-1], shape, cos, sin)
                inputs.append(y)
            for l in reversed(range(start, end)):
                _, saved = layer_forward(_lw(params, l), inputs[l - start], shape, cos, sin)
                dx, g = layer_backward(_lw(params, l), saved, dx, shape, cos, sin)
                for k2, val in g.items():
                    grads[f"layers.{l}.{k2}"] = val
    else:
        raise ValueError(mode)
    grads["embed"] = embed_backward(dx, ids, shape.vocab)
    return loss, grads


def adam_update(p, m, v, g, step, lr, beta1, beta2, eps):
    """One Adam update (bias-corrected, eps outside the square root, no
    weight decay): m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2;
    p = p - lr * (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps)."""
    dt = p.dtype.type
    m = dt(beta1) * m + dt(1 - beta1) * g
    v = dt(beta2) * v + dt(1 - beta2) * (g * g)
    mhat = m / dt(1 - beta1 ** step)
    vhat = v / dt(1 - beta2 ** step)
    p = p - dt(lr) * mhat / (np.sqrt(vhat) + dt(eps))
    return p, m, v


def train_step(params, ids, shape, state=None, step=1, mode="resident",
               ckpt_interval=None):
    """Forward, loss, backward and CPU Adam for every tensor.

    ``state`` maps name -> (m, v); zeros when None.  Returns
    (loss, grads, new_params, new_state)."""
    loss, grads = loss_and_grads(params, ids, shape, mode, ckpt_interval)
    new_params, new_state = {}, {}
    for n, p in params.items():
        if state is None:
            m = np.zeros_like(p)
            v = np.zeros_like(p)
        else:
            m, v = state[n]
        new_params[n], m2, v2 = adam_update(p, m, v, grads[n], step, shape.lr,
                                            shape.beta1, shape.beta2, shape.adam_eps)
        new_state[n] = (m2, v2)
    return loss, grads, new_params, new_state


# --------------------------------------------------------------------------
# bfloat16 (the dtype of streamed weights and offloaded gradients)
# --------------------------------------------------------------------------


def bf16_bits(x):
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    The upper 16 bits of the float32 pattern after adding 0x7FFF plus the
    lowest kept bit; NaNs map to a quiet NaN with the sign kept."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = np.where(nan, ((u >> 16) & 0x8000) | 0x7FC0, r)
    return r.astype(np.uint16)


def bf16_round(x):
    """Values of x rounded to bfloat16 (RNE), returned as float32."""
    b = bf16_bits(x).astype(np.uint32) << 16
    return b.view(np.float32)
