"""CPU oracle for the layer-streamed training step (test infrastructure only).

This package is a plain, slow NumPy statement of what one training step of
the memory-centric layer-streaming trainer computes (MegaTrain, "Full
Precision Training of 100B+ Parameter Large Language Models on a Single GPU":
Abstract; the blog summary's sections 1-4).  It exists so that tests, the
smoke check and the benchmark's CPU baseline can check the GPU library
against an independent result.  Nothing in the product path may import it,
and it imports nothing from the product: the two share only the seeded
input generators in ``synth``.

Every function is dtype-generic: float32 for parity with the GPU path,
float64 for finite-difference pins.

Parity status: every function here is pinned by CPU tests against closed
forms, invariants, library routines or the pages' printed numbers, except
the points listed as readings (the pages do not fix them).
"""
from .decoder import (  # noqa: F401
    rms_norm,
    rms_norm_backward,
    rope_cos_sin,
    rope,
    rope_backward,
    causal_attention,
    causal_attention_backward,
    silu,
    layer_forward,
    layer_backward,
    head_forward_backward,
    embed_forward,
    embed_backward,
    forward_loss,
    loss_and_grads,
    adam_update,
    train_step,
    bf16_round,
    bf16_bits,
)
