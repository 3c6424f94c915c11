"""The throughput formula and parameter count against the pages' tables."""
import os

import numpy as np

import synth
from layer_streamed_amd import metrics


def _golden(name):
    p = os.path.join(os.path.dirname(__file__), "golden", name)
    return [l.split() for l in open(p) if l.strip() and not l.startswith("#")]


QWEN7 = synth.CONFIGS["qwen2.5-7b-b16-t1024"]
QWEN14 = synth.CONFIGS["qwen2.5-14b-b8-t2048"]


def test_param_count_closed_form_matches_shapes():
    for s in list(synth.CONFIGS.values()):
        n = sum(int(np.prod(v)) for v in synth.param_shapes(s).values())
        assert metrics.shape_param_count(s) == n
    assert metrics.shape_param_count(synth.CONFIGS["tiny-2l-h256"]) == 2_491_648


def test_param_count_table5():
    for layers, billions in _golden("table5_depth.txt"):
        n = metrics.shape_param_count(QWEN7.with_(n_layers=int(layers)))
        assert round(n / 1e9, 2) == float(billions)


def test_formula_reproduces_table7():
    n = metrics.shape_param_count(QWEN7)
    for ctx, bs, step, tf in _golden("table7_long_context.txt"):
        f = metrics.formula_flops(n, QWEN7.n_layers, QWEN7.hidden, int(bs), int(ctx))
        got = metrics.tflops(f, float(step))
        assert abs(got - float(tf)) / float(tf) < 0.011, (ctx, got, tf)
    # the two longest rows pin it to the printed digit
    for ctx, bs, step, tf in _golden("table7_long_context.txt")[-2:]:
        f = metrics.formula_flops(n, QWEN7.n_layers, QWEN7.hidden, int(bs), int(ctx))
        assert round(metrics.tflops(f, float(step)), 1) == float(tf)


def test_batch_scaled_variant_does_not_fit_table7():
    n = metrics.shape_param_count(QWEN7)
    ctx, bs, step, tf = _golden("table7_long_context.txt")[1]  # 32K, BS 6
    f = metrics.formula_flops_xbatch(n, QWEN7.n_layers, QWEN7.hidden, int(bs), int(ctx))
    assert abs(metrics.tflops(f, float(step)) - float(tf)) / float(tf) > 0.3


def test_tokens_per_second_table9():
    shapes = {"qwen2.5-7b": QWEN7, "qwen2.5-14b": QWEN14}
    for model, tf, tps in _golden("table9_a6000.txt"):
        n = metrics.shape_param_count(shapes[model])
        assert abs(6 * n * float(tps) / 1e12 - float(tf)) / float(tf) < 1e-3


def _plan_ops(s, keep):
    from layer_streamed_amd import mt
    st, ops, loads, n_slots = mt.debug_plan(s.n_layers, s.ckpt_interval, 2, keep, 0)
    assert st == 0
    return ops


def _hand(s, n_fwd, n_bwd, recompute, gu_recompute):
    """Executed FLOPs by hand: every weight matrix of a layer is used in one
    product per token in the forward and two in the backward (2 FLOPs per
    multiply-add), i.e. 2*D*(P_layer - 2H) forward; attention's causal
    pairs T(T+1)/2 per sequence and head, 2*d FLOPs per pair per product,
    2 products forward and 7 backward; the head's 3 products over V x H."""
    D, H, F, d = s.tokens, s.hidden, s.ffn, s.head_dim
    mats = metrics.layer_param_count(H, s.q_dim, s.kv_dim, F) - 2 * H
    pp = 2 * d * s.batch * s.n_heads * s.seq * (s.seq + 1) / 2
    fwd = 2 * D * mats + 2 * pp
    bwd = 4 * D * mats + 7 * pp
    rec = fwd - 2 * D * F * H  # no down projection in the recompute
    gu = 2 * D * H * 2 * F
    head = 6 * D * H * s.vocab
    return (n_fwd * fwd + n_bwd * bwd + (n_bwd * rec if recompute else 0)
            + (n_bwd * gu if gu_recompute else 0) + head)


def test_executed_flops_walks_the_plan():
    s = QWEN7  # L 28, K 4
    cases = [
        # (K, keep, forward-type ops, recompute in each backward)
        (4, 1, 28 + 24, False),  # forward + re-forward of 6 segments x 4 layers
        (4, 0, 28 + 21, True),   # re-forward of the first 3 of each of 7 segments
        (1, 0, 28 + 0, True),
        (1, 1, 28 + 27, False),  # every segment but the last re-forwards its layer
    ]
    for K, keep, n_fwd, rec in cases:
        sk = s.with_(ckpt_interval=K)
        ops = _plan_ops(sk, keep)
        c = metrics.op_counts(ops)
        assert c.get(metrics.OP_FWD, 0) + c.get(metrics.OP_FWDK, 0) + c.get(
            metrics.OP_REFWD, 0) == n_fwd, (K, keep, c)
        assert c[metrics.OP_BWD] == 28 and c[metrics.OP_HEAD] == 1
        got = metrics.executed_flops(sk, ops, keep)
        want = _hand(sk, n_fwd, 28, rec, False)
        assert abs(got - want) / want < 1e-12, (K, keep, got, want)
    # the benchmark's schedule: 52 layer forwards, 28 backwards, the head
    e = metrics.executed_flops(s, _plan_ops(s, 1), 1)
    assert abs(e / 1e12 - 896.2) < 0.5, e / 1e12


def test_executed_flops_chunked_mlp_recomputes_gate_up():
    s = synth.CONFIGS["qwen2.5-7b-b1-t32768"]  # MLP over 4096-token chunks
    ops = _plan_ops(s, 1)
    got = metrics.executed_flops(s, ops, 1)
    want = _hand(s, 52, 28, False, True)
    assert abs(got - want) / want < 1e-12
    ops0 = _plan_ops(s, 0)
    assert abs(metrics.executed_flops(s, ops0, 0) - _hand(s, 49, 28, True, False)) < 1e-3 * want
