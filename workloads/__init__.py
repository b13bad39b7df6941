"""Seeded synthetic inputs for the routed MoE FFN under W4A16.

This package is shared by the float64 oracle's tests and by the HIP path's
tests and benchmark. It only draws random numbers, rounds them to the storage
formats (fp16 activations, int8/int4 codes with fp16 group scales) and packs
bytes; it holds none of the layer's own arithmetic (no dequantisation, no
projections, no routing).
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Dims,
    Weights,
    Case,
    make_config,
    make_case,
    make_weights,
    make_x,
    pack_int4,
    f16_bits,
    NEAR_TIE_FILE,
)
