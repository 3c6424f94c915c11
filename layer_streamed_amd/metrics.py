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


def executed_flops(s):
    """FLOPs one streamed step runs on the GPU: forward, segment re-forward,
    per-layer recompute and backward of every layer, plus the head.  GEMMs
    count 2*M*N*K; causal attention counts half of the full score matrix
    (forward 2 products, backward 5 products of the standard scheme)."""
    L, K = s.n_layers, s.ckpt_interval
    D, T, B = s.tokens, s.seq, s.batch
    P_mat = (s.hidden * s.q_dim + 2 * s.hidden * s.kv_dim + s.q_dim * s.hidden
             + 3 * s.hidden * s.ffn)
    gemm_fwd = 2.0 * D * P_mat
    attn_fwd = 2 * 2.0 * B * s.n_heads * s.head_dim * T * T / 2  # causal half
    layer_fwd = gemm_fwd + attn_fwd
    layer_bwd = 2 * gemm_fwd + 2.5 * attn_fwd
    # layers run forward once, the non-last members of each segment once more
    # (segment re-forward), every layer once more inside recompute, then bwd
    n_reforward = sum(min(K, L - s0) - 1 for s0 in range(0, L, K))
    layers = (L + n_reforward + L) * layer_fwd + L * layer_bwd
    head = 3 * 2.0 * D * s.hidden * s.vocab
    return layers + head


def tflops(flops, seconds):
    return flops / seconds / 1e12
