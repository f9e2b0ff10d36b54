"""Seeded synthetic inputs shared by the oracle and the HIP path.

This package holds only workload definitions and random draws (Gaussian
tokens plus a smooth 3D sinusoidal positional term, rounded to bf16).  It
contains none of the method's arithmetic: no permutation, pooling, scoring,
selection or attention.
"""
from .configs import CONFIGS, Config, get_config
from .gen import (Inputs, make_inputs, bf16_bits_to_f32, f32_to_bf16_bits, stripe_params,
                  flow_sigmas, cluster_seeds, cluster_labels)

__all__ = ["CONFIGS", "Config", "get_config", "Inputs", "make_inputs",
           "bf16_bits_to_f32", "f32_to_bf16_bits", "stripe_params", "flow_sigmas",
           "cluster_seeds", "cluster_labels"]
