"""Seeded synthetic workloads for the INSTANT low-rank backward of a linear layer.

This module only describes shapes and draws input tensors. It holds none of the
method's arithmetic (no projection, statistic, decomposition or truncation), so
both the CPU oracle and the GPU library can be fed from it without sharing code.

Shapes follow the layers the INSTANT notes evaluate on ("INSTANT: Compressing
Gradients and Activations for Resource-Efficient Training", sections 实验关键数据
and 关键发现: BERT-base blocks with L=512 tokens, EfficientFormer-L1's last stage
with 7x7=49 tokens), plus a tiny correctness case and an LLM MLP case. The token
spectra imitate the concentration the notes report (about 6 ranks holding 95% of
a BERT output gradient's energy, section 关键发现).
"""
from .configs import WORKLOADS, Workload, LayerShape, Recipe, get_workload
from .gen import (make_x, make_gy, make_w, make_layer_batch, to_io, io_to_f64,
                  bf16_bits_from_f64, bf16_bits_to_f64, sha256_of)

__all__ = ["WORKLOADS", "Workload", "LayerShape", "Recipe", "get_workload",
           "make_x", "make_gy", "make_w", "make_layer_batch", "to_io", "io_to_f64",
           "bf16_bits_from_f64", "bf16_bits_to_f64", "sha256_of"]
