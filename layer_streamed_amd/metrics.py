"""Throughput accounting for the layer-streamed training step (host logic).

Parameter count of the pre-norm GQA decoder (no biases, untied head):
  P_layer = H*Q + 2*H*Kv + Q*H + 3*H*F + 2*H,  N = L*P_layer + 2*V*H + H.
Sustained TFLOPS follows the caption of the MegaTrain page's Table 7
("Long-context training performance on GH200"): 6*N*D + 12*L*H*T^2 with
D = B*T tokens and the T^2 term not multiplied by the batch, which is how the
table's 256K and 512K rows evaluate it.  The batch-multiplied variant and the
FLOPs the streamed step actually executes are reported beside it.
"""
from __future__ import annotations


def layer_param_count(hidden, q_dim, kv_dim, ffn):
    H, Q, Kv, F = hidden, q_dim, kv_dim, ffn
    return H * Q + 2 * H * Kv + Q * H + 3 * H * F + 2 * H


def param_count(n_layers, hidden, q_dim, kv_dim, ffn, vocab):
    return (n_layers * layer_param_count(hidden, q_dim, kv_dim, ffn)
            + 2 * vocab * hidden + hidden)


def shape_param_count(s):
    return param_count(s.n_layers, s.hidden, s.q_dim, s.kv_dim, s.ffn, s.vocab)


def formula_flops(n_params, n_layers, hidden, batch, seq):
    """6*N*D + 12*L*H*T^2 (Table 7 caption), T^2 term not scaled by batch."""
    D = batch * seq
    return 6.0 * n_params * D + 12.0 * n_layers * hidden * float(seq) ** 2


def formula_flops_xbatch(n_params, n_layers, hidden, batch, seq):
    """Variant with the attention term scaled by the batch."""
    D = batch * seq
    return 6.0 * n_params * D + 12.0 * n_layers * hidden * float(seq) ** 2 * batch


# Compute-op kinds of the engine's plan (mt_debug_plan): forward, head,
# segment re-forward, (recompute +) backward, forward keeping internals.
OP_FWD, OP_HEAD, OP_REFWD, OP_BWD, OP_FWDK = 0, 1, 2, 3, 4


def _layer_flops(s):
    """Per-layer pieces of executed work: GEMMs count 2*M*N*K; attention
    counts 2*head_dim FLOPs per causal score pair (T*(T+1)/2 per sequence
    and query head) per product, forward 2 products (S, P V), backward 7
    (dK/dV kernel: S, dP, dV, dK; dQ kernel: S, dP, dQ)."""
    D, H, F = s.tokens, s.hidden, s.ffn
    nqkv = s.q_dim + 2 * s.kv_dim
    pairs = s.batch * s.n_heads * s.seq * (s.seq + 1) / 2
    pp = 2.0 * s.head_dim * pairs  # one product over the causal pairs
    g_qkv = 2.0 * D * H * nqkv
    g_o = 2.0 * D * s.q_dim * H
    g_gu = 2.0 * D * H * 2 * F
    g_down = 2.0 * D * F * H
    fwd = g_qkv + g_o + g_gu + g_down + 2 * pp
    return {
        "fwd": fwd,
        # recompute inside mt_layer_recompute_bwd: the forward without the
        # down projection (its output is not needed)
        "recompute": g_qkv + g_o + g_gu + 2 * pp,
        # backward: two products per weight (input and weight gradients)
        "bwd": 2 * (g_qkv + g_o + g_gu + g_down) + 7 * pp,
        # a chunked MLP with kept internals recomputes each chunk's gate/up
        "gu": g_gu,
    }


def executed_flops(s, ops, keep_internals=1):
    """FLOPs the streamed step runs on the GPU, walking the engine's plan
    (``ops``: (kind, layer, ...) rows of mt_debug_plan for the same depth,
    checkpoint interval and keep_internals).  A backward op recomputes its
    layer's forward unless internals are kept; with kept internals and a
    chunked MLP it still recomputes the gate/up products."""
    lf = _layer_flops(s)
    chunked = 0 < s.mlp_chunk_tokens < s.tokens
    head = 3 * 2.0 * s.tokens * s.hidden * s.vocab
    total = 0.0
    for op in ops:
        kind = int(op[0])
        if kind in (OP_FWD, OP_REFWD, OP_FWDK):
            total += lf["fwd"]
        elif kind == OP_HEAD:
            total += head
        elif kind == OP_BWD:
            total += lf["bwd"]
            if not keep_internals:
                total += lf["recompute"]
            elif chunked:
                total += lf["gu"]
        else:
            raise ValueError(f"unknown plan op kind {kind}")
    return total


def op_counts(ops):
    """Number of plan ops of each kind: {kind: count}."""
    out = {}
    for op in ops:
        out[int(op[0])] = out.get(int(op[0]), 0) + 1
    return out


def tflops(flops, seconds):
    return flops / seconds / 1e12
