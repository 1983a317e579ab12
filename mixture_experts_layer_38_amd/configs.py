"""The five MoE-layer workloads this library is measured and checked on.

Each entry fixes the layer shape (tokens T, model width d, experts E, top-K,
expert hidden width F), the arithmetic type, the routing skew applied through
the per-expert logit offset, the capacity rule and the seed of the synthetic
inputs.  Shapes follow the Mixtral-8x7B and DeepSeek-V3 routed-expert layers
that the MoE inference engineering page (ybb.press) names in its introduction
and in its §3.2; the capacity rule follows the capacity-factor definition of
the cf-1.com MoE notes, §3.1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens routed in one forward pass
    d: int            # d_model
    E: int            # number of routed experts
    K: int            # experts per token
    F: int            # expert SwiGLU hidden width (d_ff)
    dtype: str        # "f32" or "bf16": activations and weights
    skew: str = "none"        # "none" | "zipf" | "uniform": per-expert logit offset
    zipf_s: float = 0.0       # exponent of the Zipf rank law for skew == "zipf"
    bias_lo: float = 0.0      # range of the uniform per-expert bias for skew == "uniform"
    bias_hi: float = 0.0
    capacity_factor: float | None = None  # None: no per-expert cap
    alpha: float | None = None            # bias-update step (one step per pass)
    seed: int = 0
    description: str = field(default="", compare=False)

    @property
    def capacity(self) -> int:
        """Per-expert kept-row cap C = floor(cf * T * K / E), or -1 when unlimited."""
        if self.capacity_factor is None:
            return -1
        return int(math.floor(self.capacity_factor * self.T * self.K / self.E))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS: dict[str, MoEConfig] = {
    "tiny_fp32": MoEConfig(
        "tiny_fp32", T=64, d=128, E=8, K=2, F=256, dtype="f32",
        description="tiny fp32 layer, no capacity limit, lower index wins ties"),
    "mixtral_decode": MoEConfig(
        "mixtral_decode", T=32, d=4096, E=8, K=2, F=14336, dtype="bf16",
        description="Mixtral-8x7B-shaped decode step, unbiased router"),
    "mixtral_prefill": MoEConfig(
        "mixtral_prefill", T=8192, d=4096, E=8, K=2, F=14336, dtype="bf16",
        skew="zipf", zipf_s=1.2,
        description="Mixtral-8x7B-shaped prefill, Zipf(1.2) logit offset"),
    "dsv3_routed": MoEConfig(
        "dsv3_routed", T=4096, d=7168, E=256, K=8, F=2048, dtype="bf16",
        skew="uniform", bias_lo=-0.5, bias_hi=0.5,
        description="DeepSeek-V3-shaped routed experts, U(-0.5,0.5) expert bias"),
    "capacity_top2": MoEConfig(
        "capacity_top2", T=16384, d=2048, E=64, K=2, F=1408, dtype="bf16",
        skew="zipf", zipf_s=1.0, capacity_factor=1.0, alpha=1e-3,
        description="capacity-limited top-2, Zipf(1.0) offset, one bias update"),
}

# Order used when a list is wanted (smallest first).
CONFIG_ORDER = ["tiny_fp32", "mixtral_decode", "mixtral_prefill", "dsv3_routed", "capacity_top2"]


def scaled(cfg: MoEConfig, **overrides) -> MoEConfig:
    """A copy of `cfg` with some fields replaced (used for reduced-size parity cases)."""
    d = {k: getattr(cfg, k) for k in cfg.__dataclass_fields__}
    d.update(overrides)
    return MoEConfig(**d)
