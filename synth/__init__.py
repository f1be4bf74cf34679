"""Seeded synthetic inputs shaped like the LLM layers that rotation preprocessing targets.

This package is shared by the tests, the benchmark and the CPU oracle's callers.
It holds random draws and the construction of realistic tensors (Student-t
activations with outlier channels, SwiGLU products, post-RoPE queries and keys,
weights with sparse large entries) and nothing of the rotation or the
quantizer.
"""
from .inputs import (  # noqa: F401
    WORKLOADS,
    Workload,
    gaussian,
    make_inputs,
    permutation,
    r1_activations,
    r3_query_key,
    r4_activations,
    rademacher,
    tiny_activations,
    weight_with_outliers,
)
