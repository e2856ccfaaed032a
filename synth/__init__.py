"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package draws random numbers and shapes them into the workloads of the
selective-scan pages; it holds none of the scan's arithmetic, so both the fp64
oracle and the HIP path can consume its arrays without sharing any code.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_complex,
    make_complex_dense,
    make_pd,
    make_real,
    make_impulse,
    widen,
)
