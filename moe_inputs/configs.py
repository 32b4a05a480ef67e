"""Named, frozen shapes of the synthetic sparse-MoE layers.

Each entry is a layer shape taken from the model families the source pages
discuss (page "Mixture of experts: how MoE works and what it costs", sections
on loaded versus active parameters and on batching; page "Mixture of Experts:
why a model with 671 billion parameters uses only 37", sections on where MoE
changes the Transformer and on shared/fine-grained experts), made concrete with
sizes, dtypes, seeds and bias recipes.  This module holds data only.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class MoEConfig:
    """Shape and recipe of one synthetic MoE layer.

    dtype      'f32' or 'bf16': storage type of x and of every weight.
    bias       'none' | 'zipf' | 'normal': per-expert router logit bias recipe.
    bias_var   variance of the 'normal' bias.
    zipf_s     exponent of the Zipf target load for 'zipf'.
    t_sweep    token counts the layer is run at (the first T rows of one draw).
    margin     minimum gap between consecutive top-(k+1) router logits that a
               token must have to be kept (measured on the stored inputs in
               fp64); rows that miss it are replaced by the next row of the
               stream.  0 disables the filter.
    table      name of the stored row/bias table, or None when the caller
               filters rows itself.
    """

    name: str
    config_id: int
    T: int
    d: int
    E: int
    k: int
    ffn: int
    n_shared: int = 0
    ffn_shared: int = 0
    dtype: str = "bf16"
    bias: str = "none"
    bias_var: float = 0.0
    zipf_s: float = 0.0
    t_sweep: Tuple[int, ...] = ()
    seed: int = 0
    margin: float = 1e-3
    table: Optional[str] = None

    @property
    def groups(self) -> int:
        return self.E + self.n_shared

    @property
    def t_max(self) -> int:
        return max((self.T,) + tuple(self.t_sweep))

    def with_T(self, T: int) -> "MoEConfig":
        return replace(self, T=T)

    def expert_params(self) -> int:
        """Weights of one routed SwiGLU expert (three matrices)."""
        return 3 * self.d * self.ffn

    def flops(self, T: Optional[int] = None) -> int:
        """Algorithmic FLOPs of one forward: router GEMM plus two FLOPs per
        touched weight per (token, expert) pair."""
        T = self.T if T is None else T
        return (2 * T * self.d * self.E + 6 * self.d * self.ffn * T * self.k
                + 6 * self.d * self.ffn_shared * T * self.n_shared)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


TINY_F32 = MoEConfig(
    name="tiny_f32", config_id=1, T=64, d=256, E=8, k=2, ffn=512,
    dtype="f32", table="tiny_f32")

MIXTRAL = MoEConfig(
    name="mixtral", config_id=2, T=4096, d=4096, E=8, k=2, ffn=14336,
    dtype="bf16", t_sweep=(16, 4096), table="mixtral")

MIDSIZE_ZIPF = MoEConfig(
    name="midsize_zipf", config_id=3, T=8192, d=2048, E=32, k=2, ffn=1024,
    dtype="bf16", bias="zipf", zipf_s=1.1, table="midsize_zipf")

DEEPSEEK_V3 = MoEConfig(
    name="deepseek_v3", config_id=4, T=4096, d=7168, E=256, k=8, ffn=2048,
    n_shared=1, ffn_shared=2048, dtype="bf16", bias="normal", bias_var=0.5,
    table="deepseek_v3")

GPT_OSS = MoEConfig(
    name="gpt_oss", config_id=5, T=512, d=2880, E=128, k=4, ffn=2880,
    dtype="bf16", t_sweep=(1, 8, 32, 128, 512), table="gpt_oss")

NAMED = {c.name: c for c in (TINY_F32, MIXTRAL, MIDSIZE_ZIPF, DEEPSEEK_V3, GPT_OSS)}


def get(name: str) -> MoEConfig:
    return NAMED[name]
