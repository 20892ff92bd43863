"""Seeded synthetic inputs for the ZONOS2 MoE feed-forward layer.

This package only draws random numbers and rounds them to the storage type.
It holds none of the layer's arithmetic, so both the fp64 oracle and the HIP
library can consume its arrays without sharing any computation.
"""

from .configs import WORKLOADS, LayerConfig, get_config  # noqa: F401
from .gen import make_inputs, round_to_bf16_bits, bf16_bits_to_f32  # noqa: F401
