"""Layer shapes and workloads of the MoE feed-forward layer.

The model shapes are those of Table 2 in the talk notes on "Demystifying the
Mixture of Experts Serving Tax" (section "評価対象モデル (Table 2)"): hidden size,
MoE intermediate size, routed experts, experts per token and shared experts.
The token counts, routing laws and dtypes are the workloads this library is
measured on; they are synthetic (no trained weights or routing traces).

This module holds shapes only: no arithmetic of the method.
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class LayerShape:
    name: str
    hidden: int            # H
    inter: int             # I, routed expert intermediate size
    experts: int           # E
    topk: int              # K
    shared_inter: int      # I_s, total width of the shared-expert SwiGLU (0 = none)
    dtype: str             # "bf16" or "f32": storage type of x and weights
    tokens: Tuple[int, ...]
    routing: Tuple[str, ...]   # "uniform" (logits ~ N(0,1)) and/or "zipf"
    zipf_s: float = 1.2
    note: str = ""

    @property
    def dense_fa_inter(self) -> int:
        """DenseFA width: the FFN whose per-token FLOPs equal the MoE layer's.

        Definition of DenseFA (talk notes, section "定義"): the MoE layer is
        replaced by an FFN whose intermediate size is scaled by top-K; shared
        experts run on every token, so their width is added.
        """
        return self.topk * self.inter + self.shared_inter

    @property
    def dense_pa_inter(self) -> int:
        """DensePA width: a dense FFN holding as many parameters as the MoE."""
        return self.experts * self.inter + self.shared_inter


CONFIGS = {
    "tiny": LayerShape(
        name="tiny", hidden=128, inter=256, experts=8, topk=2, shared_inter=0,
        dtype="f32", tokens=(64,), routing=("uniform",),
        note="tiny MoE FFN, fp32 storage; the oracle finishes it in well under a second"),
    "mixtral": LayerShape(
        name="mixtral", hidden=4096, inter=14336, experts=8, topk=2, shared_inter=0,
        dtype="bf16", tokens=(32, 1024), routing=("uniform",),
        note="Mixtral-8x7B-shaped layer: decode T=32, prefill T=1024"),
    "qwen2": LayerShape(
        name="qwen2", hidden=3584, inter=2560, experts=64, topk=8, shared_inter=8 * 2560,
        dtype="bf16", tokens=(1, 32, 256, 2048), routing=("zipf",),
        note="Qwen2-MoE-shaped layer; 8 shared experts as one dense SwiGLU of width 20480"),
    "deepseek_v3": LayerShape(
        name="deepseek_v3", hidden=7168, inter=2048, experts=256, topk=8, shared_inter=2048,
        dtype="bf16", tokens=(128,), routing=("uniform", "zipf"),
        note="DeepSeek-V3-shaped layer; one layer's routed weights are ~22.5 GB"),
    "mixtral_sweep": LayerShape(
        name="mixtral_sweep", hidden=4096, inter=14336, experts=8, topk=2, shared_inter=0,
        dtype="bf16", tokens=(1, 8, 32, 128, 512, 2048), routing=("uniform",),
        note="MoE vs DenseFA (inter 2x14336) tax sweep"),
}

# Table 2 of the talk notes, as printed there (model name -> shape columns).
TABLE2 = {
    "Mixtral-8x7B": dict(hidden=4096, moe_inter=14336, routed=8, active=2, shared=0),
    "Qwen2-MoE": dict(hidden=3584, moe_inter=2560, routed=64, active=8, shared=8),
    "DeepSeek-V3": dict(hidden=7168, moe_inter=2048, routed=256, active=8, shared=1),
}
