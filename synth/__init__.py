"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This package holds only workload shapes and random draws: no step of the
training method (no normalisation, attention, loss, gradient or optimizer
arithmetic) lives here, so that the oracle and the HIP path can both take
their inputs from it without sharing any computation.
"""
from .inputs import (  # noqa: F401
    ModelShape,
    CONFIGS,
    param_names,
    param_shapes,
    layer_param_names,
    make_weights,
    make_tokens,
)
