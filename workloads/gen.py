"""Seeded generators for x [B,L,Cx], gy [B,L,Cy] and w [Cy,Cx].

Every draw comes from ``numpy.random.default_rng(SeedSequence([cfg, layer,
tensor, batch]))`` with tensor 0 = x, 1 = gy, 2 = w and batch = 1000 for a basis
shared by all batches. Values are built in float64 and rounded once to the I/O
dtype; the rounded bytes are what both the library and the oracle receive.

bf16 values travel as their raw 16-bit patterns (``uint16``); rounding from
float64 goes through float32 (numpy's round-to-nearest-even) and then to bf16 by
round-to-nearest-even on the bit pattern.
"""
from __future__ import annotations

import hashlib

import numpy as np
from scipy.special import erf

from .configs import Recipe, Workload

TENSOR_X, TENSOR_GY, TENSOR_W = 0, 1, 2
SHARED_BASIS_BATCH = 1000


def _rng(wl: Workload, layer_id: int, tensor: int, batch: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wl.cfg_id, layer_id, tensor, batch]))


def _profile(rec: Recipe) -> np.ndarray:
    i = np.arange(rec.rank, dtype=np.float64)
    if rec.spectrum == "pow2":
        e = 2.0 ** (-i)
    elif rec.spectrum == "geom0.6":
        e = 0.6 ** i
    elif rec.spectrum == "power1.5":
        e = (i + 1.0) ** (-1.5)
    elif rec.spectrum == "exp6":
        e = np.exp(-i / 6.0)
    else:
        raise ValueError(rec.spectrum)
    return e ** 0.25 if rec.energy_share else e


def _orthonormal(rng: np.random.Generator, L: int, r: int) -> np.ndarray:
    q, _ = np.linalg.qr(rng.standard_normal((L, r)))
    return q


def _draw(wl: Workload, layer_id: int, tensor: int, batch: int, C: int, rec: Recipe) -> np.ndarray:
    B, L = wl.B, wl.L
    if rec.rank > L:
        raise ValueError("rank exceeds token count")
    d = _profile(rec)
    if rec.scale == "unit_rms":
        d = d * np.sqrt(L / np.sum(d * d))
    rng = _rng(wl, layer_id, tensor, batch)
    if rec.per_sample:
        U = np.stack([_orthonormal(rng, L, rec.rank) for _ in range(B)])      # [B, L, r]
        V = rng.standard_normal((B, rec.rank, C))
        t = np.matmul(U * d[None, None, :], V)
    else:
        U = _orthonormal(_rng(wl, layer_id, tensor, SHARED_BASIS_BATCH), L, rec.rank)
        V = rng.standard_normal((B, rec.rank, C))
        t = np.matmul((U * d[None, :])[None], V)
    if rec.noise_var > 0.0:
        t += np.sqrt(rec.noise_var) * rng.standard_normal((B, L, C))
    if rec.gelu:
        t = 0.5 * t * (1.0 + erf(t / np.sqrt(2.0)))
    return t


def make_x(wl: Workload, layer=0, batch: int = 0) -> np.ndarray:
    """float64 x [B, L, Cx] before rounding to the I/O dtype."""
    ly = wl.layer(layer)
    return _draw(wl, ly.layer_id, TENSOR_X, batch, ly.Cx, wl.x_recipe)


def make_gy(wl: Workload, layer=0, batch: int = 0) -> np.ndarray:
    """float64 gy [B, L, Cy] before rounding to the I/O dtype."""
    ly = wl.layer(layer)
    return _draw(wl, ly.layer_id, TENSOR_GY, batch, ly.Cy, wl.gy_recipe)


def make_w(wl: Workload, layer=0) -> np.ndarray:
    """float64 w [Cy, Cx] before rounding to the I/O dtype."""
    ly = wl.layer(layer)
    rng = _rng(wl, ly.layer_id, TENSOR_W, 0)
    return wl.w_sd(ly.Cx) * rng.standard_normal((ly.Cy, ly.Cx))


# ----------------------------------------------------------------------------- dtype plumbing

def bf16_bits_from_f64(a: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    out = ((u + (((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_io(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once to the I/O dtype: float32 array, or bf16 bits as uint16."""
    if dtype == "fp32":
        return np.ascontiguousarray(a, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f64(a)
    raise ValueError(dtype)


def io_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of I/O-dtype data."""
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    raise ValueError(dtype)


def make_layer_batch(wl: Workload, layer=0, batch: int = 0, with_w: bool = False):
    """I/O-dtype x and gy of one batch (and w), plus their exact float64 values."""
    x = to_io(make_x(wl, layer, batch), wl.dtype)
    gy = to_io(make_gy(wl, layer, batch), wl.dtype)
    out = {"x": x, "gy": gy, "x64": io_to_f64(x, wl.dtype), "gy64": io_to_f64(gy, wl.dtype)}
    if with_w:
        w = to_io(make_w(wl, layer), wl.dtype)
        out["w"] = w
        out["w64"] = io_to_f64(w, wl.dtype)
    return out


def sha256_of(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode() + str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()
