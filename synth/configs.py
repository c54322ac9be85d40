"""Workloads: the five seeded synthetic MoE layers and scaled-down variants.

Shapes follow public model families' routed-expert layers.  The pages measure
on no dataset; every input is drawn here from fixed seeds.
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cfg_id: int          # seeds every tensor of this workload
    fmt: str             # "bf16" | "mxfp8" | "mxfp4" | "nvfp4"
    T: int               # tokens
    H: int               # hidden
    I: int               # intermediate (per expert)
    E: int               # routed experts
    top_k: int
    num_shared: int = 0  # always-selected experts with weight 1
    routing: str = "softmax_normal"
    x_std: float = 1.0
    w_std: float = 0.02
    zipf_s: float = 1.2

    @property
    def slots(self):
        return self.T * (self.top_k + self.num_shared)

    @property
    def flops(self):
        """Algorithmic FLOPs of the two grouped GEMMs: 6 * S * H * I."""
        return 6 * self.slots * self.H * self.I


CONFIGS = {
    # 64 tokens, hidden 256, intermediate 512, 8 experts, top-2, BF16.
    "tiny_bf16": MoEConfig("tiny_bf16", 1, "bf16", 64, 256, 512, 8, 2,
                           routing="softmax_normal"),
    # Mixtral-8x7B-shaped layer, BF16.
    "mixtral_bf16": MoEConfig("mixtral_bf16", 2, "bf16", 4096, 4096, 14336, 8, 2,
                              routing="softmax_uniform"),
    # DeepSeek-V3-shaped layer, MXFP8 weights and activations, 1 shared expert.
    "dsv3_mxfp8": MoEConfig("dsv3_mxfp8", 3, "mxfp8", 8192, 7168, 2048, 256, 8,
                            num_shared=1, routing="sigmoid_normal"),
    # Decode-shaped layer, MXFP4 weights with MXFP8 activations (W4A8).
    # T is one of DECODE_TOKENS.
    "decode_mxfp4": MoEConfig("decode_mxfp4", 4, "mxfp4", 256, 4096, 1536, 128, 8,
                              routing="softmax_uniform"),
    # NVFP4 layer under Zipf(1.2)-skewed routing.
    "nvfp4_zipf": MoEConfig("nvfp4_zipf", 5, "nvfp4", 16384, 2048, 768, 64, 6,
                            routing="zipf"),
}

DECODE_TOKENS = (1, 8, 32, 128, 256)


def scaled(name, **kw):
    """A scaled-down variant of a workload (same format, routing kind and
    seeds family) for parity tests the oracle finishes in seconds."""
    base = CONFIGS[name]
    return replace(base, name=base.name + "_small", **kw)
