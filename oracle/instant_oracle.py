"""Plain, slow, float64 CPU oracle of the INSTANT low-rank backward for y = x @ w.T.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module. It shares no code with the GPU library
and never imports it.

Source: the notes "INSTANT: Compressing Gradients and Activations for
Resource-Efficient Training" (papernotes.org, ICLR 2026). Sections cited below:
  [Framework]  整体框架   - forward unchanged, x_hat = P x stored, P/Q refreshed every N_t steps
  [KD1]        关键设计 1 - per-tensor autocorrelations C_X = E[x x^T], C_G = E[g_y g_y^T],
                             decomposed without folding in the batch; statistics only are accumulated
  [KD2]        关键设计 2 - energy threshold k, oversampling p, the Q equation (energy compensation)
  [KD3]        关键设计 3 - reordered low-rank products for g_w and g_x, and the FLOP counts

Notation: x [B, L, Cx], gy [B, L, Cy], w [Cy, Cx], P [Rx, L], Q [Ry, L].
All arithmetic is float64; inputs are the I/O-dtype values upcast exactly.

Readings where the notes leave a step open (each one also listed in the design notes):
  * sigma_i are the singular values of the symmetric PSD matrix C (= |eigenvalues|),
    so the energy is sum(sigma_i^2) = ||C||_F^2, which is the identity [KD2] states.
  * E[.] is the mean over samples; the channel sum sits inside x_b x_b^T.
  * k is the smallest index (1-based) whose prefix energy is >= eps * E ("not less than").
  * R = min(k + p, L).
  * compensation: "paper" c = (sum_{i<=R} sigma_i^2)^(-1/2) as printed in [KD2];
    "none" c = 1; "ratio" c = (E / sum_{i<=R} sigma_i^2)^(1/2). P = c * U_R^T.
  * eps is the float32 value the library receives, upcast: float64(float32(eps)).
  * g_y is projected by P for g_w and by Q for g_x ([KD3] equations).

What pins each function to something other than itself (tests/pins.py; every check
also catches a planted mistake in tests/test_oracle_mutations.py):
  eps_as_f32               float32(0.95) = 15938355 / 2^24 written out, and two golden
                           spectra whose k differs between float32(0.95) and 0.95
  Accumulator,
  autocorr_entries         element-wise loop definition; sampled entries vs the full sum
  canonical_signs          hand-built columns with ties and a zero column (golden)
  spectrum                 eigen invariants; closed-form Hadamard spectrum
  truncate                 exact rational brute force on golden and random dyadic spectra
  margin                   hand-computed golden margins; moving the threshold by less than
                           the margin keeps k, by a little more changes it (brute force)
  compensation,
  build_projection         hand-built spectrum values; P P^T = c^2 I
  calibrate_side,
  calibrate                through C = H diag(lam) H^T; exact low-rank recovery
  compress, backward       R = L identity (exact gradients); unreordered projector form
                           with unrelated P and Q; product count against the FLOP formula
  dense_projector_backward the same projector form written with einsum
  exact_backward           element-wise loop definition of g_w and g_x
  flops_*                  the 192/7 ratio of the BERT-block example ([KD3])
No function is left unpinned.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "OK", "E_ARG", "E_SHAPE", "E_STATE", "E_RANK", "E_ENERGY", "E_NONFINITE", "E_NOCONV",
    "COMP_PAPER", "COMP_NONE", "COMP_RATIO",
    "Accumulator", "autocorr_entries", "spectrum", "truncate", "compensation", "build_projection",
    "calibrate_side", "calibrate", "compress", "backward", "dense_projector_backward",
    "exact_backward", "flops_lowrank_formula", "flops_vanilla_formula", "FlopCounter",
    "canonical_signs", "eps_as_f32", "margin",
]

# status codes of the calibration (same meaning as the library's)
OK, E_ARG, E_SHAPE, E_STATE, E_RANK, E_ENERGY, E_NONFINITE, E_NOCONV = 0, 1, 2, 3, 4, 5, 6, 7
COMP_PAPER, COMP_NONE, COMP_RATIO = 0, 1, 2


def eps_as_f32(eps: float) -> float:
    """The threshold as the library sees it: a float32, upcast exactly."""
    return float(np.float32(eps))


# ----------------------------------------------------------------------------- [KD1] statistics

class Accumulator:
    """Running sum of t_b t_b^T over samples, for one tensor ([KD1]).

    Only the L x L sum and the sample count are kept; batches are never stored.
    """

    def __init__(self, L: int):
        self.L = L
        self.S = np.zeros((L, L), dtype=np.float64)
        self.n = 0

    def add(self, t: np.ndarray) -> None:
        t = np.asarray(t, dtype=np.float64)
        if t.ndim != 3 or t.shape[1] != self.L:
            raise ValueError("expected [B, L, C]")
        for b in range(t.shape[0]):
            self.S += t[b] @ t[b].T
        self.n += t.shape[0]

    def mean(self) -> np.ndarray:
        """C = E[t t^T], the mean over the samples seen."""
        return self.S / self.n


def autocorr_entries(batches, rows, cols) -> np.ndarray:
    """Selected entries C[rows[m], cols[m]] of C = E[t t^T] ([KD1]), each computed from
    its definition: the mean over samples of the channel dot product of two token rows.
    For sizes where the full L x L statistic is too large for the oracle."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    acc = np.zeros(rows.shape[0], dtype=np.float64)
    n = 0
    for t in batches:
        t = np.asarray(t, dtype=np.float64)
        for b in range(t.shape[0]):
            acc += np.einsum("mc,mc->m", t[b, rows, :], t[b, cols, :])
        n += t.shape[0]
    return acc / n


# ----------------------------------------------------------------------------- [KD1]/[KD2] decomposition

def canonical_signs(U: np.ndarray) -> np.ndarray:
    """Flip each column so that its largest-magnitude entry (lowest index on ties) is positive."""
    U = np.array(U, dtype=np.float64, copy=True)
    idx = np.argmax(np.abs(U), axis=0)
    s = np.sign(U[idx, np.arange(U.shape[1])])
    s[s == 0] = 1.0
    return U * s[None, :]


def spectrum(C: np.ndarray):
    """Singular values (descending) and left singular vectors of the symmetric PSD C.

    For a symmetric matrix the singular values are the magnitudes of the eigenvalues
    and the left singular vectors are its eigenvectors; LAPACK's symmetric
    eigensolver provides both. Columns of U follow sigma's order.
    """
    C = np.asarray(C, dtype=np.float64)
    lam, V = np.linalg.eigh(C)
    sigma = np.abs(lam)
    order = np.argsort(-sigma, kind="stable")
    return sigma[order], canonical_signs(V[:, order])


def truncate(sigma: np.ndarray, eps: float, p: int):
    """Energy-threshold truncation with oversampling ([KD2]).

    Returns (status, k, R, prefix) where prefix[j-1] = sum_{i<=j} sigma_i^2 is an
    ordered float64 running sum and E = prefix[-1]. k is the smallest j in [1, L]
    with prefix[j-1] >= eps * E; R = min(k + p, L). E == 0 gives E_ENERGY.
    """
    sigma = np.asarray(sigma, dtype=np.float64)
    L = sigma.shape[0]
    if not np.all(np.isfinite(sigma)):
        return E_NONFINITE, 0, 0, None
    prefix = np.empty(L, dtype=np.float64)
    run = 0.0
    for j in range(L):
        run += sigma[j] * sigma[j]
        prefix[j] = run
    E = prefix[-1]
    if E == 0.0:
        return E_ENERGY, 0, 0, prefix
    thr = eps * E
    k = 0
    for j in range(L):
        if prefix[j] >= thr:
            k = j + 1
            break
    R = min(k + int(p), L)
    return OK, k, R, prefix


def compensation(prefix: np.ndarray, R: int, mode: int) -> float:
    """Scalar energy compensation applied to the kept bases ([KD2], the Q equation)."""
    S_R = prefix[R - 1]
    E = prefix[-1]
    if mode == COMP_PAPER:
        return float(S_R ** -0.5)
    if mode == COMP_NONE:
        return 1.0
    if mode == COMP_RATIO:
        return float((E / S_R) ** 0.5)
    raise ValueError(mode)


def build_projection(U: np.ndarray, R: int, c: float) -> np.ndarray:
    """P = c * U_R^T, shape [R, L]: the first R left singular vectors as rows ([KD2])."""
    return c * np.ascontiguousarray(U[:, :R].T)


def margin(prefix: np.ndarray, k: int, eps: float) -> float:
    """Distance of the threshold from the two prefix sums that decide k, relative to E."""
    E = prefix[-1]
    thr = eps * E
    below = prefix[k - 2] if k >= 2 else 0.0
    return float(min(abs(prefix[k - 1] - thr), abs(below - thr)) / E)


def calibrate_side(C: np.ndarray, eps: float, p: int, comp: int, R_max: int):
    """One projection (P from C_X or Q from C_G): decomposition, truncation, compensation."""
    C = np.asarray(C, dtype=np.float64)
    if not np.all(np.isfinite(C)):
        return {"status": E_NONFINITE}
    sigma, U = spectrum(C)
    st, k, R, prefix = truncate(sigma, eps_as_f32(eps), p)
    if st != OK:
        return {"status": st, "sigma": sigma}
    if R > R_max:
        return {"status": E_RANK, "sigma": sigma, "k": k, "R": R}
    c = compensation(prefix, R, comp)
    P = build_projection(U, R, c)
    E = prefix[-1]
    gap = (sigma[R - 1] - sigma[R]) / sigma[0] if R < sigma.shape[0] else 1.0
    return {"status": OK, "sigma": sigma, "U": U, "k": k, "R": R, "c": c, "P": P,
            "E": E, "kept": prefix[R - 1] / E, "kept_k": prefix[k - 1] / E,
            "margin": margin(prefix, k, eps_as_f32(eps)), "gap": gap}


def calibrate(x_batches, gy_batches, eps: float, p: int, comp: int = COMP_PAPER, R_max: int = None):
    """Full calibration of P (from x) and Q (from gy) over the given batches ([KD1], [KD2])."""
    xa = gya = None
    for x in x_batches:
        if xa is None:
            xa = Accumulator(x.shape[1])
        xa.add(x)
    for g in gy_batches:
        if gya is None:
            gya = Accumulator(g.shape[1])
        gya.add(g)
    L = xa.L
    if R_max is None:
        R_max = L
    return {"x": calibrate_side(xa.mean(), eps, p, comp, R_max),
            "g": calibrate_side(gya.mean(), eps, p, comp, R_max),
            "C_X": xa.mean(), "C_G": gya.mean(), "n_x": xa.n, "n_g": gya.n}


# ----------------------------------------------------------------------------- [Framework]/[KD3] hot path

class FlopCounter:
    """Counts 2*M*N*K for every matrix product the oracle's backward performs."""

    def __init__(self):
        self.terms = {}

    def mm(self, name: str, a: np.ndarray, b: np.ndarray) -> np.ndarray:
        m, k = a.shape
        k2, n = b.shape
        assert k == k2
        self.terms[name] = self.terms.get(name, 0) + 2 * m * n * k
        return a @ b

    @property
    def total(self) -> int:
        return sum(self.terms.values())


def compress(P: np.ndarray, x: np.ndarray, flops: FlopCounter = None) -> np.ndarray:
    """Forward activation compression x_hat_b = P x_b, [B, Rx, Cx] ([Framework], [KD3])."""
    P = np.asarray(P, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    fc = flops or FlopCounter()
    return np.stack([fc.mm("compress", P, x[b]) for b in range(x.shape[0])])


def backward(P: np.ndarray, Q: np.ndarray, xhat: np.ndarray, gy: np.ndarray, w: np.ndarray,
             flops: FlopCounter = None):
    """Low-rank backward by the reordered products of [KD3].

    Pgy_b = P gy_b       (the transpose of gy_b^T P^T)
    Qgy_b = Q gy_b       (g_hat_y2)
    g_w   = sum_b Pgy_b^T x_hat_b
    gxh_b = Qgy_b w      (g_hat_x)
    g_x_b = Q^T gxh_b    (g_tilde_x)
    """
    P = np.asarray(P, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    xhat = np.asarray(xhat, dtype=np.float64)
    gy = np.asarray(gy, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    fc = flops or FlopCounter()
    B = gy.shape[0]
    Pgy = np.stack([fc.mm("proj_p", P, gy[b]) for b in range(B)])
    Qgy = np.stack([fc.mm("proj_q", Q, gy[b]) for b in range(B)])
    Rx, Cy = Pgy.shape[1], Pgy.shape[2]
    Cx = xhat.shape[2]
    # g_w is one contraction over the B*Rx rank-reduced rows
    gw = fc.mm("gw", Pgy.reshape(B * Rx, Cy).T, xhat.reshape(B * Rx, Cx))
    gxh = np.stack([fc.mm("gxh", Qgy[b], w) for b in range(B)])
    gx = np.stack([fc.mm("expand", Q.T, gxh[b]) for b in range(B)])
    return {"Pgy": Pgy, "Qgy": Qgy, "gw": gw, "gxh": gxh, "gx": gx}


def dense_projector_backward(P: np.ndarray, Q: np.ndarray, x: np.ndarray, gy: np.ndarray, w: np.ndarray):
    """The same approximation written with explicit L x L projectors, before any reordering:
    g_w = sum_b gy_b^T (P^T P) x_b and g_x_b = (Q^T Q) gy_b w  ([KD3])."""
    P = np.asarray(P, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    gy = np.asarray(gy, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    PtP = P.T @ P
    QtQ = Q.T @ Q
    gw = sum(gy[b].T @ (PtP @ x[b]) for b in range(x.shape[0]))
    gx = np.stack([(QtQ @ gy[b]) @ w for b in range(gy.shape[0])])
    return {"gw": gw, "gx": gx}


def exact_backward(x: np.ndarray, gy: np.ndarray, w: np.ndarray):
    """Full-rank gradients of y = x w^T: g_w = sum_b gy_b^T x_b, g_x = gy w."""
    x = np.asarray(x, dtype=np.float64)
    gy = np.asarray(gy, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    gw = sum(gy[b].T @ x[b] for b in range(x.shape[0]))
    gx = np.stack([gy[b] @ w for b in range(gy.shape[0])])
    return {"gw": gw, "gx": gx}


def flops_vanilla_formula(L: int, Cx: int, Cy: int) -> int:
    """Per-sample FLOPs of the full-rank g_w and g_x ([KD3])."""
    return 4 * L * Cx * Cy


def flops_lowrank_formula(L: int, Cx: int, Cy: int, Rx: int, Ry: int) -> int:
    """Per-sample FLOPs of the low-rank path, forward compression included ([KD3])."""
    return 2 * (Rx + Ry) * (Cx * Cy + L * Cx + L * Cy)
