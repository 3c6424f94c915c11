"""Hybrid 8-bit Adam with fast gradient clipping (test oracle).

LazyTrain (the layer-streaming optimization layer summarised on the listing
pages, in its abstract) couples 8-bit optimizer states with fast gradient
clipping in one "Hybrid 8-bit" operator: compressing the states cuts
optimizer-state memory, and the clipping is made cheap so that it offsets
the extra CPU work of the compressed update.  The page names no format and
no formula, so this module writes out the plainest reading (each point is
also listed in the design notes as a reading, not a fact of the pages):

* Format.  Each Adam moment is stored per tensor in blocks of BLOCK = 128
  consecutive elements (a tensor's last block may be shorter) as 8-bit
  floating-point codes of the OCP FP8 E4M3 format -- 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits, subnormals, no infinities, largest
  finite magnitude 448, codes 0x7F / 0xFF are NaN -- with one fp32 scale
  per block: scale = absmax(block) / 448, code = E4M3(x * (448 / absmax))
  rounded to nearest, ties to even (values just above 448 from the rounding
  of the factor saturate to 448), value = E4M3value(code) * scale.  A block
  of zeros has scale 0 and zero codes.
* What is stored.  The first moment m as is; the second moment v as its
  square root r = sqrt(v) (the format then covers v over twice the
  exponent range), read back as v = r * r.
* "Hybrid".  The fp32 master weights stay fp32; the update is computed in
  fp32 from the dequantized old moments and the new gradient, with the
  same operations as the fp32 Adam (PyTorch semantics, ``decoder.adam_update``),
  and the new moments are quantized after the update.
* Clipping.  Every gradient is multiplied by c = min(1, max_norm / (norm +
  1e-6)), norm = the L2 norm of the whole model's gradient (the usual
  global-norm clipping of LLM training); "fast": the product applies c
  inside the update pass, so clipping costs no pass of its own over the
  gradients (the norm itself is accumulated where the gradients are made).

All arithmetic of an update is fp32 (numpy float32), in the order written,
so that an implementation evaluating the same operations gets bitwise the
same result.

Test infrastructure only: nothing in the product may import this module.
"""
from __future__ import annotations

import numpy as np

from .decoder import loss_and_grads

BLOCK = 128
E4M3_MAX = 448.0


def e4m3_value(codes):
    """float32 values of OCP E4M3 codes (uint8): E = bits 6..3, M = bits
    2..0; E > 0: 2^(E-7) (1 + M/8); E = 0: 2^-6 M/8; E = 15, M = 7: NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    mag = np.where(E > 0, np.ldexp(1.0 + M / 8.0, E - 7), np.ldexp(M / 8.0, -6))
    out = sign * mag
    out = np.where((E == 15) & (M == 7), np.nan, out)
    return out.astype(np.float32)


def e4m3_code(x):
    """OCP E4M3 codes of float32 values, rounded to nearest (ties to even),
    finite magnitudes above 448 saturated to 448.  NaN is not expected here
    (the optimizer refuses non-finite gradients)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)  # exact
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.abs(x)
    f, k = np.frexp(a)  # a = f 2^k, f in [0.5, 1): exponent e = k - 1, a = (2f) 2^e
    e = k - 1
    normal = a >= 2.0 ** -6
    # normal range: mantissa steps of 2^(e-3); subnormal range: steps of 2^-9
    step_exp = np.where(normal, e - 3, -9)
    q = np.rint(np.ldexp(a, -step_exp)).astype(np.int64)  # ties to even
    # normal: q in [8, 16] -> E = e + 7 (+1 if q == 16); subnormal: q in [0, 8]
    E = np.where(normal, e + 7, 0)
    M = np.where(normal, q - 8, q)
    carry = np.where(normal, q == 16, q == 8)
    E = np.where(carry, E + 1, E)
    M = np.where(carry, 0, M)
    over = (E > 15) | ((E == 15) & (M == 7))
    E = np.where(over, 15, E)
    M = np.where(over, 6, M)
    return (sign | (E << 3) | M).astype(np.uint8)


def blocks(n):
    """[lo, hi) ranges of a tensor of n elements' quantization blocks."""
    return [(lo, min(n, lo + BLOCK)) for lo in range(0, n, BLOCK)]


def quantize(x):
    """Block-scaled E4M3 of a flat float32 array: (codes uint8 [n], scales
    float32 [n_blocks])."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    codes = np.zeros(x.size, np.uint8)
    scales = np.zeros(len(blocks(x.size)), np.float32)
    for b, (lo, hi) in enumerate(blocks(x.size)):
        amax = np.max(np.abs(x[lo:hi]))
        if amax == 0:
            continue
        scales[b] = np.float32(amax) / np.float32(E4M3_MAX)
        codes[lo:hi] = e4m3_code(x[lo:hi] * (np.float32(E4M3_MAX) / np.float32(amax)))
    return codes, scales


def dequantize(codes, scales):
    """Values of block-scaled E4M3 codes (float32 [n])."""
    vals = e4m3_value(codes)
    out = np.empty(vals.size, np.float32)
    for b, (lo, hi) in enumerate(blocks(vals.size)):
        out[lo:hi] = vals[lo:hi] * np.float32(scales[b])
    return out


def zero_state(n):
    """The 8-bit state of a fresh tensor: all moments zero."""
    nb = len(blocks(n))
    return (np.zeros(n, np.uint8), np.zeros(nb, np.float32),
            np.zeros(n, np.uint8), np.zeros(nb, np.float32))


def adam8_update(p, state, g, step, lr, beta1, beta2, eps, clip=1.0):
    """One hybrid 8-bit Adam update of a flat fp32 tensor.

    state = (m codes, m scales, r codes, r scales) with r = sqrt(v).
    Returns (new p, new state).  ``clip`` multiplies the gradient first."""
    f = np.float32
    p = np.asarray(p, np.float32).reshape(-1)
    g = np.asarray(g, np.float32).reshape(-1) * f(clip)
    mc, ms, rc, rs = state
    m_old = dequantize(mc, ms)
    r_old = dequantize(rc, rs)
    v_old = r_old * r_old
    m = f(beta1) * m_old + f(1 - beta1) * g
    v = f(beta2) * v_old + f(1 - beta2) * (g * g)
    mhat = m / f(1 - beta1 ** step)
    vhat = v / f(1 - beta2 ** step)
    p = p - f(lr) * mhat / (np.sqrt(vhat) + f(eps))
    r = np.sqrt(v)
    return p, quantize(m) + quantize(r)


def clip_coefficient(grads, max_norm):
    """c = min(1, max_norm / (norm + 1e-6)) with norm the L2 norm over every
    tensor (float64 sum of squares), as an fp32 factor; 1 when max_norm is
    0 (clipping off)."""
    if max_norm <= 0:
        return np.float32(1.0)
    ss = sum(float(np.sum(np.asarray(g, np.float64) ** 2)) for g in grads.values())
    return np.float32(min(1.0, max_norm / (np.sqrt(ss) + 1e-6)))


def train_step_adam8(params, ids, shape, state=None, step=1, max_norm=0.0,
                     mode="resident", ckpt_interval=None):
    """Forward, loss, backward, global-norm clipping and the hybrid 8-bit
    Adam for every tensor.  ``state`` maps name -> 8-bit state (zero when
    None).  Returns (loss, grads, clip factor, new params, new state)."""
    loss, grads = loss_and_grads(params, ids, shape, mode, ckpt_interval)
    c = clip_coefficient(grads, max_norm)
    new_p, new_s = {}, {}
    for n, p in params.items():
        st = zero_state(p.size) if state is None else state[n]
        q, s2 = adam8_update(p, st, grads[n], step, shape.lr, shape.beta1, shape.beta2,
                             shape.adam_eps, c)
        new_p[n] = q.reshape(p.shape)
        new_s[n] = s2
    return loss, grads, c, new_p, new_s
