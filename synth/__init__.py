"""Seeded synthetic inputs for the EAGLE-3 draft-and-verify path.

This package only draws random numbers with fixed shapes and distributions.
It holds none of the method's arithmetic, so both the CPU oracle and the HIP
path can be fed from it without sharing any computation.
"""
from .gen import (CONFIGS, Config, config, weights, seq_inputs, prefix_kv,
                  contexts, target_noise, uniforms, seed_features, normal,
                  uniform_ints, GenKey)

__all__ = ["CONFIGS", "Config", "config", "weights", "seq_inputs", "prefix_kv",
           "contexts", "target_noise", "uniforms", "seed_features", "normal",
           "uniform_ints", "GenKey"]
