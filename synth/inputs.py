"""Workload shapes and seeded random draws (weights, token ids).

Shapes follow the Qwen2.5-shaped decoders of the MegaTrain page (Table 2,
"Model configurations used in experiments"; Table 6 for the 2.0x width point)
and the small parity model.  Every parameter is named here once, so that the
oracle, the C library's host store and the tests agree on names and shapes.

Draws: each matrix is an independent stream ``default_rng([seed, i])`` of
float64 standard normals scaled by ``std`` and cast to float32, where ``i`` is
the tensor's index in ``param_names`` order.  Norm gains start at 1.  Token ids
are uniform in ``[0, vocab)`` from ``default_rng([token_seed])``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "ModelShape",
    "CONFIGS",
    "param_names",
    "param_shapes",
    "layer_param_names",
    "make_weights",
    "make_tokens",
]


@dataclass(frozen=True)
class ModelShape:
    """Decoder shape plus the per-step workload (batch, sequence, knobs)."""

    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    batch: int = 1
    seq: int = 1
    ckpt_interval: int = 4
    mlp_chunk_tokens: int = 0  # 0 = whole token set in one MLP pass
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    adam_eps: float = 1e-8
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def with_(self, **kw) -> "ModelShape":
        return replace(self, **kw)


# The workloads.  Names say what each one is.
CONFIGS: dict[str, ModelShape] = {
    # Small parity model: 2 layers, hidden 256, GQA 4/2, head_dim 64.
    "tiny-2l-h256": ModelShape(
        name="tiny-2l-h256", n_layers=2, hidden=256, n_heads=4, n_kv_heads=2,
        head_dim=64, ffn=1024, vocab=1024, batch=2, seq=128, ckpt_interval=1),
    # Qwen2.5-7B shape, B 16 x T 1024, checkpoint every 4 layers.
    "qwen2.5-7b-b16-t1024": ModelShape(
        name="qwen2.5-7b-b16-t1024", n_layers=28, hidden=3584, n_heads=28,
        n_kv_heads=4, head_dim=128, ffn=18944, vocab=152064, batch=16,
        seq=1024, ckpt_interval=4),
    # Qwen2.5-14B shape, B 8 x T 2048.
    "qwen2.5-14b-b8-t2048": ModelShape(
        name="qwen2.5-14b-b8-t2048", n_layers=48, hidden=5120, n_heads=40,
        n_kv_heads=8, head_dim=128, ffn=13824, vocab=152064, batch=8,
        seq=2048, ckpt_interval=4),
    # 2.0x width point: hidden 7168, FFN 37888, 8 layers, B 8 x T 1024.
    "width2x-8l-b8-t1024": ModelShape(
        name="width2x-8l-b8-t1024", n_layers=8, hidden=7168, n_heads=56,
        n_kv_heads=8, head_dim=128, ffn=37888, vocab=152064, batch=8,
        seq=1024, ckpt_interval=4),
    # Qwen2.5-7B shape at 32K context, B 1, MLP over 4096-token chunks.
    "qwen2.5-7b-b1-t32768": ModelShape(
        name="qwen2.5-7b-b1-t32768", n_layers=28, hidden=3584, n_heads=28,
        n_kv_heads=4, head_dim=128, ffn=18944, vocab=152064, batch=1,
        seq=32768, ckpt_interval=4, mlp_chunk_tokens=4096),
    # 128K, 256K and 512K context, the pages' ultra-long-context range (Table 7)
    "qwen2.5-7b-b1-t131072": ModelShape(
        name="qwen2.5-7b-b1-t131072", n_layers=28, hidden=3584, n_heads=28,
        n_kv_heads=4, head_dim=128, ffn=18944, vocab=152064, batch=1,
        seq=131072, ckpt_interval=4, mlp_chunk_tokens=4096),
    "qwen2.5-7b-b1-t262144": ModelShape(
        name="qwen2.5-7b-b1-t262144", n_layers=28, hidden=3584, n_heads=28,
        n_kv_heads=4, head_dim=128, ffn=18944, vocab=152064, batch=1,
        seq=262144, ckpt_interval=4, mlp_chunk_tokens=4096),
    "qwen2.5-7b-b1-t524288": ModelShape(
        name="qwen2.5-7b-b1-t524288", n_layers=28, hidden=3584, n_heads=28,
        n_kv_heads=4, head_dim=128, ffn=18944, vocab=152064, batch=1,
        seq=524288, ckpt_interval=4, mlp_chunk_tokens=4096),
    # The pages' larger dense shapes (Table 2: Qwen2.5-32B, H 5120 / F 27648,
    # 64 layers; Qwen2.5-72B, H 8192 / F 29568, 80 layers) at their full
    # width but a few layers (a host store of the whole depth would take
    # 0.45-1.0 TB); head_dim 128, 8 KV heads as in those models.
    "qwen2.5-32b-l8-b8-t1024": ModelShape(
        name="qwen2.5-32b-l8-b8-t1024", n_layers=8, hidden=5120, n_heads=40,
        n_kv_heads=8, head_dim=128, ffn=27648, vocab=152064, batch=8,
        seq=1024, ckpt_interval=4),
    "qwen2.5-72b-l4-b8-t1024": ModelShape(
        name="qwen2.5-72b-l4-b8-t1024", n_layers=4, hidden=8192, n_heads=64,
        n_kv_heads=8, head_dim=128, ffn=29568, vocab=152064, batch=8,
        seq=1024, ckpt_interval=4),
}

# The width study (Table 6): the 7B-shaped layer scaled to 1.5x .. 3.5x
# hidden and FFN size at head_dim 128 with GQA groups of 7 as in the 7B
# shape, B 8 x T 1024.  A few layers each (the host store of 28 such
# layers would take up to 1.1 TB); the 2.0x point is width2x-8l-b8-t1024.
for _scale, _h, _f, _L in (("1.5x", 5376, 28416, 4), ("2.5x", 8960, 47360, 4),
                           ("3.0x", 10752, 56832, 2), ("3.5x", 12544, 66304, 2)):
    _name = f"width{_scale}-{_L}l-b8-t1024"
    CONFIGS[_name] = ModelShape(
        name=_name, n_layers=_L, hidden=_h, n_heads=_h // 128, n_kv_heads=_h // 128 // 7,
        head_dim=128, ffn=_f, vocab=152064, batch=8, seq=1024, ckpt_interval=4)

# Per-layer tensors in draw order; gains ("*_norm") are not drawn.
_LAYER_TENSORS = ("attn_norm", "w_q", "w_k", "w_v", "w_o", "mlp_norm",
                  "w_gate", "w_up", "w_down")


def layer_param_names(layer: int) -> list[str]:
    return [f"layers.{layer}.{t}" for t in _LAYER_TENSORS]


def param_names(shape: ModelShape) -> list[str]:
    """All parameter names: embedding, layers in order, final norm, LM head."""
    names = ["embed"]
    for l in range(shape.n_layers):
        names += layer_param_names(l)
    names += ["final_norm", "lm_head"]
    return names


def param_shapes(shape: ModelShape) -> dict[str, tuple[int, ...]]:
    """Row-major [out, in] matrices; gains are vectors of the hidden size."""
    H, Q, Kv, F, V = shape.hidden, shape.q_dim, shape.kv_dim, shape.ffn, shape.vocab
    per_layer = {
        "attn_norm": (H,), "w_q": (Q, H), "w_k": (Kv, H), "w_v": (Kv, H),
        "w_o": (H, Q), "mlp_norm": (H,), "w_gate": (F, H), "w_up": (F, H),
        "w_down": (H, F),
    }
    out = {"embed": (V, H)}
    for l in range(shape.n_layers):
        for t in _LAYER_TENSORS:
            out[f"layers.{l}.{t}"] = per_layer[t]
    out["final_norm"] = (H,)
    out["lm_head"] = (V, H)
    return out


def _is_gain(name: str) -> bool:
    return name.endswith("norm")


def make_weights(shape: ModelShape, seed: int = 0, std: float = 0.02,
                 names: list[str] | None = None,
                 dtype=np.float32, bf16_exact: bool = False) -> dict[str, np.ndarray]:
    """Seeded weights: matrices ~ N(0, std^2), gains = 1.

    ``names`` restricts the draw to a subset (each tensor has its own stream,
    so a subset draws exactly the values the full set would).
    ``bf16_exact`` clears the low 16 bits of every float32 draw (truncation
    toward zero), so the values are exactly representable in bfloat16 and an
    fp32 master and its 16-bit copy start out equal.
    """
    shapes = param_shapes(shape)
    order = param_names(shape)
    wanted = order if names is None else list(names)
    index = {n: i for i, n in enumerate(order)}
    out: dict[str, np.ndarray] = {}
    for n in wanted:
        shp = shapes[n]
        if _is_gain(n):
            out[n] = np.ones(shp, dtype=dtype)
        else:
            rng = np.random.default_rng([seed, index[n]])
            a = (rng.standard_normal(shp) * std).astype(np.float32)
            if bf16_exact:
                a = (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
            out[n] = a.astype(dtype)
    return out


def make_tokens(shape: ModelShape, seed: int = 1, batch: int | None = None,
                seq: int | None = None) -> np.ndarray:
    """Uniform token ids in [0, vocab), int32, shape [batch, seq]."""
    B = shape.batch if batch is None else batch
    T = shape.seq if seq is None else seq
    rng = np.random.default_rng([seed])
    return rng.integers(0, shape.vocab, size=(B, T), dtype=np.int64).astype(np.int32)
