"""Seeded synthetic inputs for the DECO MoE feed-forward layer.

This package only draws random numbers and rounds them to the storage type.
It holds none of the layer's arithmetic, so both the fp64 oracle (through the
tests) and the HIP library (through the tests and the benchmark) can be fed
from it without sharing any computation.
"""
from .gen import (CONFIGS, LayerInputs, make_layer, make_custom, make_dout, round_to_bf16,
                  bf16_bits, dense_equivalent_dff)

__all__ = ["CONFIGS", "LayerInputs", "make_layer", "make_custom", "make_dout", "round_to_bf16",
           "bf16_bits", "dense_equivalent_dff"]
