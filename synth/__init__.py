"""Seeded synthetic inputs for the fused-MoE path.

This module only draws and packs input data; it holds none of the method's
arithmetic.  Tests, ``bench.py`` and ``smoke()`` take their inputs from here,
so the oracle and the HIP path see identical bits.

Host-side draws use ``numpy.random.default_rng([config_id, tensor_id,
sub_id])`` (PCG64, seeded by the tuple); large weight tensors can instead be
drawn directly on a GPU with a seeded ``torch.Generator`` so that tens of GB
need not be generated on the host.  bfloat16 values are produced by
round-to-nearest-even from float32 and handled as raw 16-bit patterns.
"""

from .inputs import (host_rng, normal_f32, f32_to_bf16_bits, bf16_bits_to_f32,
                     zipf_group_sizes, symmetric_int8_rows, device_normal_bf16,
                     device_normal_f32)
from .configs import CONFIGS, Config

__all__ = ["host_rng", "normal_f32", "f32_to_bf16_bits", "bf16_bits_to_f32",
           "zipf_group_sizes", "symmetric_int8_rows", "device_normal_bf16",
           "device_normal_f32",
           "CONFIGS", "Config"]
