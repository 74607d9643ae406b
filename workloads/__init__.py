"""Seeded synthetic workloads for diagonal-aware sparse attention.

This package holds the workload shapes and the seeded input generators
that both the HIP library's tests/bench and the CPU oracle are fed from.
It contains none of the method's arithmetic (no keep-set rule, no
softmax): only shapes, random numbers and cache layouts.  Neither
``oracle`` nor ``ar_image_generation_amd`` imports it.
"""
from .configs import (  # noqa: F401
    BAND, CONFIGS, DENSE, MODE_NAMES, PREFILL_CONFIGS, ROWDIAG, DecodeConfig,
    PrefillConfig, get, small_decode)
from .generate import (  # noqa: F401
    DecodeInputs,
    PrefillInputs,
    correlated_field,
    decode_inputs,
    positions,
    prefill_inputs,
)
