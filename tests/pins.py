"""Checks that pin the CPU oracle to what the INSTANT notes and plain mathematics fix.

Each check takes the oracle module as an argument and raises AssertionError when
the oracle disagrees, so the same checks can run against the real oracle and
against copies with a planted mistake (see test_oracle_mutations.py).
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H / np.sqrt(n)


def random_case(seed, B=3, L=16, Cx=12, Cy=10, rank=None):
    rng = np.random.default_rng(seed)
    if rank is None:
        x = rng.standard_normal((B, L, Cx))
        gy = rng.standard_normal((B, L, Cy))
    else:
        Ux = np.linalg.qr(rng.standard_normal((L, rank)))[0]
        Ug = np.linalg.qr(rng.standard_normal((L, rank)))[0]
        x = np.einsum("lr,brc->blc", Ux, rng.standard_normal((B, rank, Cx)))
        gy = np.einsum("lr,brc->blc", Ug, rng.standard_normal((B, rank, Cy)))
    w = rng.standard_normal((Cy, Cx))
    return x, gy, w


def calibrated(O, x, gy, eps, p, comp, R_max=None):
    cal = O.calibrate([x], [gy], eps, p, comp, R_max)
    assert cal["x"]["status"] == O.OK and cal["g"]["status"] == O.OK
    return cal["x"], cal["g"]


# --------------------------------------------------------------------------- P1
def check_full_rank_identity(O, seed=0):
    """At R = L with uncompensated orthonormal P and Q, P^T P = Q^T Q = I, so the
    low-rank gradients equal the exact g_w = sum gy^T x and g_x = gy w."""
    x, gy, w = random_case(seed)
    L = x.shape[1]
    sx, sg = calibrated(O, x, gy, 0.95, L, O.COMP_NONE)
    assert sx["R"] == L and sg["R"] == L
    xh = O.compress(sx["P"], x)
    out = O.backward(sx["P"], sg["P"], xh, gy, w)
    gw_exact = np.einsum("blo,bli->oi", gy, x)
    gx_exact = np.einsum("blo,oi->bli", gy, w)
    assert rel(out["gw"], gw_exact) < 1e-12, rel(out["gw"], gw_exact)
    assert rel(out["gx"], gx_exact) < 1e-12, rel(out["gx"], gx_exact)
    # with the printed compensation, P^T P = c_P^2 I: g_w scales by c_P^2, g_x by c_Q^2
    sx2, sg2 = calibrated(O, x, gy, 0.95, L, O.COMP_PAPER)
    out2 = O.backward(sx2["P"], sg2["P"], O.compress(sx2["P"], x), gy, w)
    assert rel(out2["gw"], sx2["c"] ** 2 * gw_exact) < 1e-12
    assert rel(out2["gx"], sg2["c"] ** 2 * gx_exact) < 1e-12


# --------------------------------------------------------------------------- P2
def check_reordering(O, seed=1):
    """The reordered products equal the unreordered projector form
    g_w = sum_b gy_b^T (P^T P) x_b, g_x_b = (Q^T Q) gy_b w, for unrelated P and Q
    (so swapping P and Q, or dropping a factor, is caught)."""
    x, gy, w = random_case(seed, B=4, L=20, Cx=9, Cy=7)
    rng = np.random.default_rng(seed + 100)
    P = rng.standard_normal((5, 20))
    Q = rng.standard_normal((3, 20))
    out = O.backward(P, Q, O.compress(P, x), gy, w)
    gw_ref = np.einsum("blo,lm,bmi->oi", gy, P.T @ P, x)
    gx_ref = np.einsum("lm,bmo,oi->bli", Q.T @ Q, gy, w)
    assert rel(out["gw"], gw_ref) < 1e-12, rel(out["gw"], gw_ref)
    assert rel(out["gx"], gx_ref) < 1e-12, rel(out["gx"], gx_ref)
    # the oracle's own projector form agrees too
    dn = O.dense_projector_backward(P, Q, x, gy, w)
    assert rel(dn["gw"], gw_ref) < 1e-12 and rel(dn["gx"], gx_ref) < 1e-12
    # intermediate shapes follow the notes' notation
    assert out["Pgy"].shape == (4, 5, 7) and out["Qgy"].shape == (4, 3, 7)
    assert out["gxh"].shape == (4, 3, 9) and out["gx"].shape == (4, 20, 9)


# --------------------------------------------------------------------------- P3
def brute_force_k(sigma, eps):
    """Exact rational evaluation of the definition: smallest k with
    sum_{i<=k} sigma_i^2 >= eps * sum_i sigma_i^2."""
    sq = [Fraction(float(s)) ** 2 for s in sigma]
    E = sum(sq)
    thr = Fraction(float(np.float32(eps))) * E
    run = Fraction(0)
    for j, v in enumerate(sq):
        run += v
        if run >= thr:
            return j + 1
    raise AssertionError("unreachable")


def check_truncation_golden(O):
    g = load_golden("truncation_spectra.json")
    for case in g["cases"]:
        sigma = np.ones(64) if case["sigma"] == "ones64" else np.array(case["sigma"], dtype=np.float64)
        st, k, R, prefix = O.truncate(sigma, O.eps_as_f32(case["eps"]), case["p"])
        assert st == O.OK
        assert (k, R) == (case["k"], case["R"]), (case["name"], k, R)
        assert brute_force_k(sigma, case["eps"]) == case["k"]


def check_truncation_bruteforce(O, trials=300, seed=2):
    """Random dyadic spectra (exact in binary), random dyadic eps, brute-force k."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        L = int(rng.integers(1, 40))
        sigma = np.sort(rng.integers(0, 9, size=L).astype(np.float64) / 4.0)[::-1].copy()
        if sigma[0] == 0:
            sigma[0] = 1.0
        eps = int(rng.integers(1, 65)) / 64.0
        p = int(rng.integers(0, 5))
        st, k, R, _ = O.truncate(sigma, O.eps_as_f32(eps), p)
        assert st == O.OK
        kb = brute_force_k(sigma, eps)
        assert k == kb, (sigma, eps, k, kb)
        assert R == min(kb + p, L)


def check_truncation_through_matrix(O):
    """The same decision through C = H diag(lam) H^T (normalised Hadamard), where C is
    only approximately exact: used where the decision has a clear margin."""
    L = 32
    H = hadamard(L)
    rng = np.random.default_rng(5)
    for trial in range(20):
        lam = np.sort(rng.uniform(0.0, 1.0, L) ** 3)[::-1]
        lam[0] = 1.0
        eps = float(rng.uniform(0.5, 0.99))
        kb = brute_force_k(lam, eps)
        sq = np.cumsum(lam ** 2)
        thr = np.float32(eps) * sq[-1]
        m = min(abs(sq[kb - 1] - thr), abs((sq[kb - 2] if kb > 1 else 0.0) - thr)) / sq[-1]
        if m < 1e-3:
            continue
        C = H @ np.diag(lam) @ H.T
        s = O.calibrate_side(C, eps, 1, O.COMP_NONE, L)
        assert s["status"] == O.OK and s["k"] == kb, (trial, s["k"], kb)


def check_error_semantics(O):
    L = 8
    assert O.calibrate_side(np.zeros((L, L)), 0.95, 2, O.COMP_PAPER, L)["status"] == O.E_ENERGY
    C = np.eye(L)
    C[3, 3] = np.nan
    assert O.calibrate_side(C, 0.95, 2, O.COMP_PAPER, L)["status"] == O.E_NONFINITE
    # flat spectrum: k = ceil(0.95 * 8) = 8, R = 8 > R_max = 4
    assert O.calibrate_side(np.eye(L), 0.95, 0, O.COMP_PAPER, 4)["status"] == O.E_RANK


# --------------------------------------------------------------------------- P4
def check_flop_formula(O):
    g = load_golden("flop_ratio_bert_block.json")
    v = O.flops_vanilla_formula(g["L"], g["Cx"], g["Cy"])
    lr = O.flops_lowrank_formula(g["L"], g["Cx"], g["Cy"], g["Rx"], g["Ry"])
    assert Fraction(v, lr) == Fraction(g["exact_ratio_num"], g["exact_ratio_den"])
    assert round(v / lr) == g["printed_ratio_approx"]
    # the products the oracle performs add up to the formula, term by term
    B, L, Cx, Cy, Rx, Ry = 3, 16, 12, 10, 5, 3
    x, gy, w = random_case(7, B, L, Cx, Cy)
    rng = np.random.default_rng(8)
    P = rng.standard_normal((Rx, L))
    Q = rng.standard_normal((Ry, L))
    fc = O.FlopCounter()
    xh = O.compress(P, x, fc)
    O.backward(P, Q, xh, gy, w, fc)
    t = fc.terms
    assert t["compress"] == B * 2 * Rx * L * Cx
    assert t["proj_p"] + t["proj_q"] == B * 2 * (Rx + Ry) * L * Cy
    assert t["gw"] == B * 2 * Rx * Cx * Cy
    assert t["gxh"] == B * 2 * Ry * Cx * Cy
    assert t["expand"] == B * 2 * Ry * L * Cx
    assert fc.total == B * O.flops_lowrank_formula(L, Cx, Cy, Rx, Ry)


# --------------------------------------------------------------------------- P5
def check_eigen_invariants(O, seed=3):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((24, 40))
    C = A @ A.T / 40.0
    sigma, U = O.spectrum(C)
    assert np.all(np.diff(sigma) <= 0)
    assert abs(sigma.sum() - np.trace(C)) < 1e-12 * np.trace(C)
    assert abs((sigma ** 2).sum() - np.sum(C * C)) < 1e-12 * np.sum(C * C)
    assert np.abs(U.T @ U - np.eye(24)).max() < 1e-12
    assert np.linalg.norm(C @ U - U * sigma[None, :]) < 1e-12 * np.linalg.norm(C)
    # closed form: known eigenvalues and eigenvectors
    L = 16
    H = hadamard(L)
    lam = 2.0 ** -np.arange(L)
    perm = np.random.default_rng(seed).permutation(L)
    C = H[:, perm] @ np.diag(lam) @ H[:, perm].T
    sigma, U = O.spectrum(C)
    assert np.abs(sigma - lam).max() < 1e-14
    assert np.abs(np.abs(U.T @ H[:, perm]) - np.eye(L)).max() < 1e-10


# --------------------------------------------------------------------------- P6
def check_exact_lowrank_recovery(O, seed=4):
    """Noise-free data in a shared rank-r token subspace with R >= r: P^T P x = x,
    Q^T Q gy = gy, so the low-rank gradients are exact."""
    rng = np.random.default_rng(seed)
    B, L, Cx, Cy, r = 4, 24, 10, 14, 5
    Ux = np.linalg.qr(rng.standard_normal((L, r)))[0]
    Ug = np.linalg.qr(rng.standard_normal((L, r)))[0]
    x = np.einsum("lr,brc->blc", Ux, rng.standard_normal((B, r, Cx)))
    gy = np.einsum("lr,brc->blc", Ug, rng.standard_normal((B, r, Cy)))
    w = rng.standard_normal((Cy, Cx))
    sx, sg = calibrated(O, x, gy, 1.0, 0, O.COMP_NONE)
    assert sx["k"] == r and sg["k"] == r
    out = O.backward(sx["P"], sg["P"], O.compress(sx["P"], x), gy, w)
    assert rel(out["gw"], np.einsum("blo,bli->oi", gy, x)) < 1e-10
    assert rel(out["gx"], np.einsum("blo,oi->bli", gy, w)) < 1e-10
    # span(P^T) = span(Ux), span(Q^T) = span(Ug)
    assert np.linalg.norm(sx["P"].T @ (sx["P"] @ Ux) - Ux) < 1e-10
    assert np.linalg.norm(sg["P"].T @ (sg["P"] @ Ug) - Ug) < 1e-10


# --------------------------------------------------------------------------- P7
def check_compensation_algebra(O, seed=6):
    x, gy, w = random_case(seed, L=16)
    for comp in (O.COMP_PAPER, O.COMP_NONE, O.COMP_RATIO):
        sx, _ = calibrated(O, x, gy, 0.8, 1, comp)
        P, c, R = sx["P"], sx["c"], sx["R"]
        assert np.abs(P @ P.T - c * c * np.eye(R)).max() < 1e-12 * max(c * c, 1.0)
        PtP = P.T @ P
        assert np.abs(PtP @ PtP - c * c * PtP).max() < 1e-12 * max(c ** 4, 1.0)
    # values of c on a hand-built spectrum: sigma^2 = 4,1,1,1,1 (E = 8) at eps = 0.625, p = 0 -> R = 2
    sigma = np.array([2.0, 1.0, 1.0, 1.0, 1.0])
    st, k, R, prefix = O.truncate(sigma, O.eps_as_f32(0.625), 0)
    assert (k, R) == (2, 2)
    assert abs(O.compensation(prefix, R, O.COMP_PAPER) - 5.0 ** -0.5) < 1e-15
    assert O.compensation(prefix, R, O.COMP_NONE) == 1.0
    assert abs(O.compensation(prefix, R, O.COMP_RATIO) - (8.0 / 5.0) ** 0.5) < 1e-15


# --------------------------------------------------------------------------- P8
def check_monotone_in_p(O, seed=9):
    """More oversampled bases never reconstruct the activations worse: the residual
    ||x - P^T P x|| is non-increasing in p (uncompensated, nested subspaces)."""
    x, gy, w = random_case(seed, B=4, L=24, Cx=16, Cy=16)
    errs = []
    for p in range(0, 10):
        sx, _ = calibrated(O, x, gy, 0.5, p, O.COMP_NONE)
        P = sx["P"]
        errs.append(np.linalg.norm(x - np.einsum("lm,bmc->blc", P.T @ P, x)))
    assert all(errs[i + 1] <= errs[i] * (1 + 1e-12) for i in range(len(errs) - 1)), errs


# --------------------------------------------------------------------------- P9
def check_memory_count(O):
    """x_hat keeps Rx of L token rows: at L=512 and Rx=16 the stored activation is 32x smaller."""
    rng = np.random.default_rng(10)
    P = rng.standard_normal((16, 512))
    x = rng.standard_normal((2, 512, 3))
    xh = O.compress(P, x)
    assert x.size / xh.size == 32.0


# --------------------------------------------------------------------------- statistics
def check_autocorrelation(O, seed=11):
    """C = E[t t^T] over samples, with the channel sum inside; order of batches is irrelevant."""
    rng = np.random.default_rng(seed)
    t1 = rng.standard_normal((3, 6, 5))
    t2 = rng.standard_normal((2, 6, 5))
    acc = O.Accumulator(6)
    acc.add(t1)
    acc.add(t2)
    ref = np.zeros((6, 6))
    for t in (t1, t2):
        for b in range(t.shape[0]):
            for i in range(6):
                for j in range(6):
                    ref[i, j] += sum(t[b, i, c] * t[b, j, c] for c in range(5))
    assert acc.n == 5
    assert np.abs(acc.mean() - ref / 5).max() < 1e-13
    assert np.allclose(acc.mean(), acc.mean().T, rtol=0, atol=0)


def check_autocorr_entries(O, seed=12):
    """Sampled entries equal the full statistic's entries (and its symmetry)."""
    rng = np.random.default_rng(seed)
    t1 = rng.standard_normal((3, 7, 4))
    t2 = rng.standard_normal((2, 7, 4))
    acc = O.Accumulator(7)
    acc.add(t1)
    acc.add(t2)
    rows = rng.integers(0, 7, 20)
    cols = rng.integers(0, 7, 20)
    got = O.autocorr_entries([t1, t2], rows, cols)
    assert np.abs(got - acc.mean()[rows, cols]).max() < 1e-13
    assert np.abs(got - O.autocorr_entries([t1, t2], cols, rows)).max() == 0.0


# --------------------------------------------------------------------------- eps as float32
def check_eps_is_float32(O):
    """The library receives eps as a float32; the oracle's threshold uses that value.
    float32(0.95) = 15938355 / 2^24 (the nearest float32 to 0.95, below it); 0.625 is exact.
    The golden spectra float32_eps_* (truncation_spectra.json) decide k differently under
    float32(0.95) and 0.95, and the truncation through calibrate_side must take the
    float32 branch too."""
    assert Fraction(O.eps_as_f32(0.95)) == Fraction(15938355, 2 ** 24)
    assert O.eps_as_f32(0.625) == 0.625
    assert O.eps_as_f32(1.0) == 1.0
    g = load_golden("truncation_spectra.json")
    cases = [c for c in g["cases"] if c["name"].startswith("float32_eps")]
    assert len(cases) == 2
    for case in cases:
        sigma = np.array(case["sigma"], dtype=np.float64)
        # C = diag(sigma) is exact, and its decomposition returns sigma itself
        s = O.calibrate_side(np.diag(sigma), case["eps"], case["p"], O.COMP_NONE, len(sigma))
        assert s["status"] == O.OK and (s["k"], s["R"]) == (case["k"], case["R"]), (case["name"], s["k"])


# --------------------------------------------------------------------------- margin of the k decision
def check_margin_golden(O):
    """Hand-computed margins (tests/golden/margin_cases.json)."""
    g = load_golden("margin_cases.json")
    for case in g["cases"]:
        sigma = np.array(case["sigma"], dtype=np.float64)
        st, k, R, prefix = O.truncate(sigma, case["eps"], 0)
        assert st == O.OK and k == case["k"], (case["name"], k)
        m = O.margin(prefix, k, case["eps"])
        assert abs(m - case["margin"]) <= 1e-15, (case["name"], m, case["margin"])


def check_margin_property(O, trials=300, seed=13):
    """What the margin means: moving the threshold by less than margin * E in either
    direction keeps k, and moving it by a little more towards the nearer deciding prefix
    sum changes k. Brute force on random dyadic spectra (exact prefix sums)."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        L = int(rng.integers(2, 30))
        sigma = np.sort(rng.integers(0, 9, size=L).astype(np.float64) / 4.0)[::-1].copy()
        sigma[0] = max(sigma[0], 1.0)
        eps = int(rng.integers(1, 64)) / 64.0 + 1.0 / 1024.0
        st, k, _, prefix = O.truncate(sigma, eps, 0)
        assert st == O.OK
        m = O.margin(prefix, k, eps)
        E = prefix[-1]
        below = prefix[k - 2] if k >= 2 else 0.0
        assert m > 0.0
        for f in (0.99, -0.99):
            e2 = eps + f * m
            if 0.0 < e2 <= 1.0:
                assert brute_force_k_f64(sigma, e2) == k, (sigma, eps, m, f)
        # the nearer side: the prefix sum S_k (threshold moving up past it changes k to k+1)
        # or S_{k-1} (threshold moving down past it changes k to k-1 or less)
        up = abs(prefix[k - 1] - eps * E) <= abs(below - eps * E)
        e2 = eps + (1.01 * m if up else -1.01 * m)
        if 0.0 < e2 <= 1.0:
            assert brute_force_k_f64(sigma, e2) != k, (sigma, eps, m)


def brute_force_k_f64(sigma, eps):
    """Smallest k with sum_{i<=k} sigma_i^2 >= eps * E, in exact rationals, eps taken as given."""
    sq = [Fraction(float(s)) ** 2 for s in sigma]
    thr = Fraction(float(eps)) * sum(sq)
    run = Fraction(0)
    for j, v in enumerate(sq):
        run += v
        if run >= thr:
            return j + 1
    raise AssertionError("unreachable")


# --------------------------------------------------------------------------- exact gradients
def check_exact_backward_loops(O, seed=14):
    """The full-rank gradients of y = x w^T from their element-wise definition:
    g_w[o][i] = sum_b sum_l gy[b][l][o] x[b][l][i] and g_x[b][l][i] = sum_o gy[b][l][o] w[o][i]
    (plain Python loops; Cx != Cy so a transposed operand cannot pass)."""
    rng = np.random.default_rng(seed)
    B, L, Cx, Cy = 2, 3, 2, 4
    x = rng.standard_normal((B, L, Cx))
    gy = rng.standard_normal((B, L, Cy))
    w = rng.standard_normal((Cy, Cx))
    gw = [[0.0] * Cx for _ in range(Cy)]
    for o in range(Cy):
        for i in range(Cx):
            for b in range(B):
                for l in range(L):
                    gw[o][i] += gy[b, l, o] * x[b, l, i]
    gx = [[[0.0] * Cx for _ in range(L)] for _ in range(B)]
    for b in range(B):
        for l in range(L):
            for i in range(Cx):
                for o in range(Cy):
                    gx[b][l][i] += gy[b, l, o] * w[o, i]
    out = O.exact_backward(x, gy, w)
    assert np.shape(out["gw"]) == (Cy, Cx) and np.shape(out["gx"]) == (B, L, Cx)
    assert np.abs(np.asarray(out["gw"]) - np.array(gw)).max() < 1e-12
    assert np.abs(np.asarray(out["gx"]) - np.array(gx)).max() < 1e-12


# --------------------------------------------------------------------------- eigenvector gauge
def check_canonical_signs_golden(O):
    """Sign rule on hand-built columns with ties and a zero column
    (tests/golden/canonical_signs.json)."""
    g = load_golden("canonical_signs.json")
    U = np.array(g["input_columns"], dtype=np.float64).T
    want = np.array(g["expected_columns"], dtype=np.float64).T
    got = O.canonical_signs(U)
    assert np.array_equal(got, want), got
    assert np.array_equal(U, np.array(g["input_columns"], dtype=np.float64).T)  # input untouched
    # spectrum() returns its vectors in that gauge
    _, V = O.spectrum(np.diag([3.0, 2.0, 1.0]) - 0.5 * np.ones((3, 3)))
    assert np.array_equal(V, O.canonical_signs(V))


ALL_CHECKS = [
    check_full_rank_identity, check_reordering, check_truncation_golden,
    check_truncation_bruteforce, check_truncation_through_matrix, check_error_semantics,
    check_flop_formula, check_eigen_invariants, check_exact_lowrank_recovery,
    check_compensation_algebra, check_monotone_in_p, check_memory_count, check_autocorrelation,
    check_autocorr_entries, check_eps_is_float32, check_margin_golden, check_margin_property,
    check_exact_backward_loops, check_canonical_signs_golden,
]
