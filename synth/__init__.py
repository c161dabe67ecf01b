"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This package only draws random tensors and rounds them to 16-bit storage
formats. It contains none of the hybrid-attention arithmetic, so both sides
can consume its output without sharing any of the method's code.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    DecodeInputs,
    PrefillInputs,
    bf16_bits_from_f32,
    f16_bits_from_f32,
    make_decode_inputs,
    make_prefill_inputs,
    make_append_tokens,
    small_decode_inputs,
)
