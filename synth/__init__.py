"""Seeded synthetic inputs shared by the GPU tests, the bench and the oracle.

This module only draws numbers and lays out structure (planted blocks,
planted needles); it performs none of the arithmetic of the attention method
itself, so the oracle and the GPU path stay independent of each other while
consuming the same input bits.
"""
from .gen import (normal, normal_np, splitmix64_np, planted_block_ids,
                  needle_positions, moba_inputs, moba_decode_inputs, esa_inputs,
                  compression_weights)

__all__ = ["normal", "normal_np", "splitmix64_np", "planted_block_ids",
           "needle_positions", "moba_inputs", "moba_decode_inputs", "esa_inputs",
           "compression_weights"]
