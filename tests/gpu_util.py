"""Helpers for the GPU tests: move I/O-dtype arrays to the device and back, and
compare against the oracle."""
import numpy as np
import torch

import workloads as W


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def from_dev(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return W.bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.float().cpu().numpy().astype(np.float64)


def empty(shape, dtype: str) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


TOL = {"fp32": 1e-4, "bf16": 2e-2}
