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


# Per-element bound beside the Frobenius one: the textbook forward error bound of a chain
# of dot products, |got - ref| <= tau * mag elementwise, where mag is the same chain of
# products computed on the absolute values of every operand (each output element's sum of
# |terms|; see oracle_magnitudes). tau counts the roundings that reach an output, in units
# of the I/O dtype's unit roundoff u:
#   bf16 (u = 2^-8): P or Q enters twice, two stored intermediates (P g_y or x_hat, Q g_y
#   and g_hat_x) and the output itself are rounded once each: 5u to first order, plus u of
#   room for the float32 accumulation (at most ~13k terms here: 13k * 2^-24 < 2^-8).
#   fp32: no intermediate rounding; the accumulation over the chain's sums (at most ~600
#   terms in the fp32 cases: 600 * 2^-24 = 3.6e-5) stays under 1e-4.
ELEM_TOL = {"fp32": 1e-4, "bf16": 6 * 2.0 ** -8}


def oracle_magnitudes(O, P, Q, x64, gy64, w64):
    """The oracle's x_hat and backward run on |P|, |Q|, |x|, |g_y|, |w|: for every output
    element the sum of the magnitudes of the products it is made of (x_hat = |P||x|;
    g_w = sum_b (|P||g_y|)^T (|P||x|); g_x = |Q|^T ((|Q||g_y|) |w|))."""
    aP, aQ = np.abs(np.asarray(P, dtype=np.float64)), np.abs(np.asarray(Q, dtype=np.float64))
    xh = O.compress(aP, np.abs(x64))
    out = O.backward(aP, aQ, xh, np.abs(gy64), np.abs(w64))
    return xh, out


def elem_err(a, b, mag) -> float:
    """Largest |a - b| / mag over the elements (mag = 0 requires a == b there)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    d = np.abs(a - b)
    zero = mag == 0.0
    if np.any(d[zero] != 0.0):
        return float("inf")
    return float(np.max(d[~zero] / mag[~zero])) if np.any(~zero) else 0.0


def check_close(name, got, ref, dtype, mag) -> str:
    """Both criteria: relative Frobenius error <= TOL and |got - ref| <= ELEM_TOL * mag."""
    e_f, e_e = rel(got, ref), elem_err(got, ref, mag)
    assert e_f <= TOL[dtype], f"{name}: relative Frobenius error {e_f:.3e} > {TOL[dtype]}"
    assert e_e <= ELEM_TOL[dtype], f"{name}: per-element error {e_e:.3e} of the term magnitudes > {ELEM_TOL[dtype]}"
    return f"{name} {e_f:.2e}/{e_e:.2e}"
