"""Seeded synthetic MoE-layer workloads shared by the tests, the oracle checks and bench.py.

This package draws inputs only: activations, router logits (or a given routing), and
stacked expert weights, already rounded to the storage formats the library consumes.
It holds none of the layer's arithmetic (no softmax, top-k, counting, permutation,
FFN or combine); those live independently in ``oracle/`` and in the HIP library.
"""
from .gen import (  # noqa: F401
    Workload,
    CONFIG_NAMES,
    SKEW_TARGETS,
    config,
    make,
    to_numpy_bits,
    with_maxvio,
)
