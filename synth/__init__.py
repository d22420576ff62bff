"""Seeded synthetic inputs for the CubicQuant dequant-GEMM workloads.

This module only draws random inputs (integer codes, scales, shape parameters,
activations, routing ids). It holds none of the method's arithmetic: it never
packs, decodes or multiplies. Both the oracle-side tests and the HIP-side
tests, bench and smoke consume what it returns.
"""
from .gen import *  # noqa: F401,F403
