"""Planted mistakes in the oracle must be caught by its pins.

Each case patches one oracle function with a plausible error (a sign, an
index, a dropped term) on the CPU and checks that at least one pin test
fails.  This shows the pins constrain the oracle, not only agree with it.
"""
import numpy as np
import pytest

from oracle import decoder as D
import tests.test_oracle_pins as P


def _rope_wrong_sign(x, cos, sin):
    half = x.shape[-1] // 2
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)


def _kv_head_modulo(h, n_heads, n_kv_heads):
    return h % n_kv_heads


def _adam_no_bias_correction(p, m, v, g, step, lr, beta1, beta2, eps):
    dt = p.dtype.type
    m = dt(beta1) * m + dt(1 - beta1) * g
    v = dt(beta2) * v + dt(1 - beta2) * (g * g)
    return p - dt(lr) * m / (np.sqrt(v) + dt(eps)), m, v


_orig_head = D.head_forward_backward


def _head_mean_over_all_positions(x, gain, w_out, ids, eps, want_logits=False):
    out = list(_orig_head(x, gain, w_out, ids, eps, want_logits))
    B, T = ids.shape
    out[0] = out[0] * (B * (T - 1)) / (B * T)
    return tuple(out)


_orig_rms = D.rms_norm


def _rms_without_eps(x, gain, eps):
    return _orig_rms(x, gain, 0.0)


MUTATIONS = [
    ("rope", _rope_wrong_sign, [P.test_rope_pairing_and_angle]),
    ("_kv_head", _kv_head_modulo, [lambda: P.test_attention_matches_sdpa_and_autograd(4, 2)]),
    ("adam_update", _adam_no_bias_correction, [P.test_adam_matches_torch_optim_adam]),
    ("head_forward_backward", _head_mean_over_all_positions,
     [lambda: P.test_head_loss_against_torch_cross_entropy(),
      lambda: P.test_against_torch_autograd_float64(P.TINY)]),
    ("rms_norm", _rms_without_eps, [lambda: P.test_against_torch_autograd_float64(P.TINY.with_(rms_eps=0.5))]),
]


@pytest.mark.parametrize("name,fn,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn, pins):
    monkeypatch.setattr(D, name, fn)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught the planted mistake in {name}"
