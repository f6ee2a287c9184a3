"""Workload definitions: layer shapes, hyper-parameters and data recipes.

Every number here is a shape, a hyper-parameter or a data-distribution parameter;
none of it is derived from the method's results (ranks are recomputed by whoever
consumes the data).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Recipe:
    """How one activation-like tensor [B, L, C] is drawn.

    t_b = scale * U_b @ diag(d) @ V_b  (+ noise)  (then optionally GELU)

    * U_b: L x r with orthonormal columns (QR of a seeded Gaussian). Shared by all
      samples (``per_sample=False``) or drawn per sample.
    * d: per-rank scale. ``spectrum`` names the profile e_i (i = 0..r-1); when
      ``energy_share`` is set, e_i is read as the share of the autocorrelation's
      squared-eigenvalue energy, so d_i = e_i ** (1/4) (the eigenvalues of
      E[t t^T] go as d_i^2, their squares as d_i^4); otherwise d_i = e_i.
    * V_b: r x C, i.i.d. N(0, 1).
    * noise: i.i.d. N(0, noise_var) added per element (a variance, not an sd).
    * scale: ``"unit_rms"`` scales so that the expected per-element mean square of
      the low-rank part is 1; ``"none"`` leaves it as drawn.
    * gelu: apply the erf-form GELU elementwise after everything else.
    """
    rank: int
    spectrum: str             # "pow2" | "geom0.6" | "power1.5" | "exp6"
    energy_share: bool
    per_sample: bool = False
    noise_var: float = 0.0
    scale: str = "unit_rms"
    gelu: bool = False


@dataclass(frozen=True)
class LayerShape:
    name: str
    layer_id: int
    Cx: int
    Cy: int


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    description: str
    B: int
    L: int
    layers: Tuple[LayerShape, ...]
    dtype: str                # "fp32" | "bf16"  (I/O dtype of x, gy, w, xhat, gw, gx)
    eps: float
    p: int
    n_cal: int
    n_t: int
    x_recipe: Recipe
    gy_recipe: Recipe
    w_std: str                # "inv_sqrt_cx" (variance 1/Cx) | "0.02"

    def layer(self, name_or_index=0) -> LayerShape:
        if isinstance(name_or_index, int):
            return self.layers[name_or_index]
        for ly in self.layers:
            if ly.name == name_or_index:
                return ly
        raise KeyError(name_or_index)

    def w_sd(self, Cx: int) -> float:
        if self.w_std == "inv_sqrt_cx":
            return 1.0 / float(Cx) ** 0.5
        return float(self.w_std)


WORKLOADS = {
    # Tiny single linear layer in fp32; spelled out fully: per-sample rank-8
    # bases, d_i = 2^-i, noise variance 1e-3, w ~ N(0, 1/Cx).
    "tiny": Workload(
        name="tiny", cfg_id=1,
        description="tiny single linear, fp32: B=2 L=64 Cx=Cy=64",
        B=2, L=64, layers=(LayerShape("main", 0, 64, 64),), dtype="fp32",
        eps=0.95, p=2, n_cal=4, n_t=100,
        x_recipe=Recipe(rank=8, spectrum="pow2", energy_share=False, per_sample=True,
                        noise_var=1e-3, scale="none"),
        gy_recipe=Recipe(rank=8, spectrum="pow2", energy_share=False, per_sample=True,
                         noise_var=1e-3, scale="none"),
        w_std="inv_sqrt_cx"),
    # BERT-base attention-projection-shaped linear, bf16 I/O.
    "bert_attn": Workload(
        name="bert_attn", cfg_id=2,
        description="BERT-base attention projection, bf16: B=32 L=512 Cx=Cy=768",
        B=32, L=512, layers=(LayerShape("main", 0, 768, 768),), dtype="bf16",
        eps=0.95, p=2, n_cal=16, n_t=100,
        x_recipe=Recipe(rank=64, spectrum="geom0.6", energy_share=True),
        gy_recipe=Recipe(rank=64, spectrum="geom0.6", energy_share=True),
        w_std="0.02"),
    # BERT-base FFN pair; x of both layers is GELU of the low-rank construction.
    "bert_ffn": Workload(
        name="bert_ffn", cfg_id=3,
        description="BERT-base FFN up 768->3072 and down 3072->768, bf16: B=32 L=512",
        B=32, L=512, layers=(LayerShape("up", 0, 768, 3072), LayerShape("down", 1, 3072, 768)),
        dtype="bf16", eps=0.95, p=8, n_cal=16, n_t=100,
        x_recipe=Recipe(rank=64, spectrum="geom0.6", energy_share=True, gelu=True),
        gy_recipe=Recipe(rank=64, spectrum="geom0.6", energy_share=True),
        w_std="0.02"),
    # EfficientFormer-L1 last-stage-shaped linears: 7x7 tokens, large batch.
    "effformer": Workload(
        name="effformer", cfg_id=4,
        description="EfficientFormer-L1 last stage 448->1792 and 1792->448, bf16: B=128 L=49",
        B=128, L=49, layers=(LayerShape("up", 0, 448, 1792), LayerShape("down", 1, 1792, 448)),
        dtype="bf16", eps=0.95, p=4, n_cal=16, n_t=100,
        x_recipe=Recipe(rank=49, spectrum="power1.5", energy_share=True),
        gy_recipe=Recipe(rank=49, spectrum="power1.5", energy_share=True),
        w_std="0.02"),
    # LLM MLP-shaped linear with a long token axis.
    "llm_mlp": Workload(
        name="llm_mlp", cfg_id=5,
        description="LLM MLP up 4096->11008, bf16: B=8 L=2048",
        B=8, L=2048, layers=(LayerShape("main", 0, 4096, 11008),), dtype="bf16",
        eps=0.95, p=16, n_cal=16, n_t=100,
        x_recipe=Recipe(rank=128, spectrum="exp6", energy_share=True, noise_var=1e-3),
        gy_recipe=Recipe(rank=128, spectrum="exp6", energy_share=True, noise_var=1e-3),
        w_std="0.02"),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]
