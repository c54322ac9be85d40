"""Seeded synthetic inputs for the fused MoE layer.

This package holds the workload definitions and the seeded generators that
both the HIP path (tests, bench) and the CPU oracle consume.  It contains
none of the layer's arithmetic: it draws float32 normals and router logits,
picks top-k experts, and casts to BF16 with torch's own conversion.
Quantising weights into MX/NVFP4 codes is done by each side separately.
"""

from .configs import CONFIGS, MoEConfig, scaled  # noqa: F401
from .gen import (  # noqa: F401
    gen_x_bf16, gen_weight_f32, gen_weight_f32_device, gen_routing,
    gen_w2_input_scale, bf16_bits,
)
