"""Layer shapes of the synthetic workloads.

The shapes follow the MoE layers the Colibri pages deploy or benchmark on:
Mixtral-8x7B (d_model 4096, 8 experts, d_ff 14336, top-2), a shared-expert
augmented fine-grained layer, a many-expert layer with skewed routing, and an
int8-weight Mixtral-8x22B-shaped decode layer (and its int4 group-wise twin),
plus a tiny fp32 layer that the oracle evaluates in full.
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str
    d_model: int
    n_experts: int
    d_ff: int
    top_k: int
    act_dtype: str            # "f32" | "bf16"
    expert_dtype: str         # "f32" | "bf16" | "i8" | "i4"
    tokens: Tuple[int, ...]   # the token counts the workload is run at
    shared_d_ff: int = 0      # 0: no shared expert
    zipf_s: float = 0.0       # >0: router bias drawn from a Zipf law over experts
    zipf_beta: float = 3.0    # bias = beta * ln p_rank
    seed: int = 0

    @property
    def has_bias(self) -> bool:
        return self.zipf_s > 0.0


CONFIGS = {
    "tiny_f32": LayerConfig("tiny_f32", 256, 8, 512, 2, "f32", "f32", (64,)),
    "mixtral_bf16": LayerConfig("mixtral_bf16", 4096, 8, 14336, 2, "bf16", "bf16",
                                (1, 8, 32, 64, 4096)),
    "shared_fine_bf16": LayerConfig("shared_fine_bf16", 3584, 64, 2560, 8, "bf16", "bf16",
                                    (16, 2048), shared_d_ff=20480),
    "skewed_bf16": LayerConfig("skewed_bf16", 2048, 128, 768, 4, "bf16", "bf16",
                               (8192,), zipf_s=1.2, zipf_beta=3.0),
    "int8_mixtral22b": LayerConfig("int8_mixtral22b", 6144, 8, 16384, 2, "bf16", "i8",
                                   (1, 16, 256)),
    # the same layer with int4 group-wise weights (group 128), the next step below int8
    "int4_mixtral22b": LayerConfig("int4_mixtral22b", 6144, 8, 16384, 2, "bf16", "i4",
                                   (1, 16, 256)),
}


def get_config(name: str, **overrides) -> LayerConfig:
    """A named config, optionally with fields replaced (for reduced-size cases)."""
    base = CONFIGS[name]
    if not overrides:
        return base
    d = dict(base.__dict__)
    d.update(overrides)
    return LayerConfig(**d)
