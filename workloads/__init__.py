"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This package only draws random numbers and rounds them to the storage dtype.
It holds none of the attention arithmetic, none of the block bookkeeping and
imports neither the GPU package nor the oracle.
"""
from .synth import (  # noqa: F401
    DTYPES,
    Workload,
    bf16_bits_from_f32,
    make_tiny,
    make_gqa70b,
    make_highbatch,
    make_long,
    make_verify,
    make_prefill,
    make_custom,
    by_name,
    with_rising_scores,
)
