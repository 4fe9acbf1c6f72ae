"""The five workloads of the fused-MoE path, with their shapes and input
recipes.  Ids double as the first element of every seed tuple."""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    T: int = 0            # tokens (or GMM rows M)
    H: int = 0            # hidden size (GMM: K)
    I: int = 0            # expert intermediate size (GMM: N)
    E: int = 0            # experts
    topk: int = 0
    groups: int = 1       # num_expert_group
    topk_group: int = 1
    renormalize: bool = True
    scale: float = 1.0    # routed_scaling_factor
    x_dtype: str = "bf16"
    w_std: float = 0.02
    extra: dict = field(default_factory=dict)


CONFIGS = {
    "tiny": Config(1, "tiny fused MoE forward", T=64, H=128, I=256, E=8,
                   topk=2, x_dtype="f32"),
    "routing": Config(2, "GroupedTopK routing", T=83, E=256, topk=8,
                      groups=8, topk_group=4),
    "prefill": Config(3, "prefill-shaped MoE layer", T=4096, H=2048, I=768,
                      E=128, topk=8),
    "decode16": Config(4, "decode-shaped MoE layer T=16", T=16, H=7168,
                       I=2048, E=256, topk=8, groups=8, topk_group=4,
                       scale=2.5),
    "decode64": Config(4, "decode-shaped MoE layer T=64", T=64, H=7168,
                       I=2048, E=256, topk=8, groups=8, topk_group=4,
                       scale=2.5, extra={"sub": 1}),
    "int8gmm": Config(5, "INT8 grouped GEMM", T=2048, H=4096, I=4096, E=32,
                      extra={"zipf_s": 1.2}),
}
