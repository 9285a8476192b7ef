"""Seeded synthetic inputs for the MoE FFN layer forward pass.

This package only draws random numbers and stores them in the layouts the
library and the oracle both read.  It holds none of the layer's arithmetic:
no routing, no softmax, no expert evaluation.  Both the HIP path and the CPU
oracle consume exactly the bits produced here.
"""
from .configs import CONFIGS, MoEConfig, get_config, custom_config  # noqa: F401
from .gen import Workload, bf16_bits_to_f32, f32_to_bf16_bits  # noqa: F401
