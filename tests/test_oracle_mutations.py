"""Plant plausible mistakes in the CPU oracle and check that some pin catches each.

Every mutation is applied with monkeypatch to the oracle module on the CPU and
undone after the test; the GPU library is not involved.
"""
import numpy as np
import pytest

import oracle as O
from oracle import instant_oracle as M
import pins


def _fails(checks):
    for chk in checks:
        try:
            chk(O)
        except Exception:
            return True
    return False


def _truncate_strict(sigma, eps, p):
    st, k, R, prefix = _ORIG_TRUNCATE(sigma, eps, p)
    if st != O.OK:
        return st, k, R, prefix
    thr = eps * prefix[-1]
    k = int(np.argmax(prefix > thr)) + 1          # '>' instead of '>='
    return st, k, min(k + p, len(prefix)), prefix


def _truncate_off_by_one(sigma, eps, p):
    st, k, R, prefix = _ORIG_TRUNCATE(sigma, eps, p)
    if st != O.OK:
        return st, k, R, prefix
    return st, max(k - 1, 1), min(max(k - 1, 1) + p, len(prefix)), prefix


def _truncate_no_oversampling(sigma, eps, p):
    st, k, R, prefix = _ORIG_TRUNCATE(sigma, eps, p)
    return st, k, k, prefix


def _truncate_energy_not_squared(sigma, eps, p):
    # energy as sum(sigma) instead of sum(sigma^2)
    return _ORIG_TRUNCATE(np.sqrt(np.abs(sigma)), eps, p)


def _spectrum_ascending(C):
    s, U = _ORIG_SPECTRUM(C)
    return s[::-1].copy(), U[:, ::-1].copy()


def _spectrum_unsorted_vectors(C):
    s, U = _ORIG_SPECTRUM(C)
    return s, U[:, ::-1].copy()


def _comp_wrong_sign(prefix, R, mode):
    if mode == O.COMP_PAPER:
        return float(prefix[R - 1] ** 0.5)
    return _ORIG_COMP(prefix, R, mode)


def _comp_uses_E(prefix, R, mode):
    if mode == O.COMP_PAPER:
        return float(prefix[-1] ** -0.5)
    return _ORIG_COMP(prefix, R, mode)


def _backward_swaps_pq(P, Q, xhat, gy, w, flops=None):
    return _ORIG_BACKWARD(Q, P, xhat, gy, w, flops) if P.shape == Q.shape else \
        _ORIG_BACKWARD(P, P[: Q.shape[0]], xhat, gy, w, flops)


def _backward_last_sample_only(P, Q, xhat, gy, w, flops=None):
    out = _ORIG_BACKWARD(P, Q, xhat, gy, w, flops)
    out["gw"] = out["Pgy"][-1].T @ xhat[-1]
    return out


def _backward_gx_without_expand_transpose(P, Q, xhat, gy, w, flops=None):
    out = _ORIG_BACKWARD(P, Q, xhat, gy, w, flops)
    out["gx"] = np.stack([Q.T @ (Q @ (Q.T @ out["gxh"][b])) for b in range(gy.shape[0])])
    return out


def _backward_gx_sign(P, Q, xhat, gy, w, flops=None):
    out = _ORIG_BACKWARD(P, Q, xhat, gy, w, flops)
    out["gx"] = -out["gx"]
    return out


def _compress_reversed_tokens(P, x, flops=None):
    # a wrong token index: P applied to the token axis in reverse order
    return _ORIG_COMPRESS(P, x[:, ::-1, :], flops)


class _AccPerChannel(M.Accumulator):
    def mean(self):
        return self.S / (self.n * 5)


def _lowrank_formula_wrong(L, Cx, Cy, Rx, Ry):
    return 2 * (Rx + Ry) * (Cx * Cy + L * Cx)


def _eps_unrounded(eps):
    # the decimal threshold instead of the float32 value the library receives
    return float(eps)


def _margin_shift_up(prefix, k, eps):
    # reads S_{k+1} and S_k instead of S_k and S_{k-1}
    E = prefix[-1]
    thr = eps * E
    nxt = prefix[k] if k < len(prefix) else prefix[-1]
    return float(min(abs(nxt - thr), abs(prefix[k - 1] - thr)) / E)


def _margin_shift_down(prefix, k, eps):
    # reads S_{k-1} and S_{k-2} instead of S_k and S_{k-1}
    E = prefix[-1]
    thr = eps * E
    a = prefix[k - 2] if k >= 2 else 0.0
    b = prefix[k - 3] if k >= 3 else 0.0
    return float(min(abs(a - thr), abs(b - thr)) / E)


def _margin_absolute(prefix, k, eps):
    # not relative to E
    return _ORIG_MARGIN(prefix, k, eps) * prefix[-1]


def _exact_gx_scaled(x, gy, w):
    out = _ORIG_EXACT(x, gy, w)
    out["gx"] = 1.5 * out["gx"]
    return out


def _exact_gw_first_sample(x, gy, w):
    out = _ORIG_EXACT(x, gy, w)
    out["gw"] = np.asarray(gy, dtype=np.float64)[0].T @ np.asarray(x, dtype=np.float64)[0]
    return out


def _signs_untouched(U):
    return np.array(U, dtype=np.float64, copy=True)


def _signs_tie_to_last(U):
    # ties of the largest magnitude go to the highest index
    U = np.array(U, dtype=np.float64, copy=True)
    a = np.abs(U)[::-1]
    idx = U.shape[0] - 1 - np.argmax(a, axis=0)
    s = np.sign(U[idx, np.arange(U.shape[1])])
    s[s == 0] = 1.0
    return U * s[None, :]


def _signs_largest_value(U):
    # the largest signed value instead of the largest magnitude
    U = np.array(U, dtype=np.float64, copy=True)
    idx = np.argmax(U, axis=0)
    s = np.sign(U[idx, np.arange(U.shape[1])])
    s[s == 0] = 1.0
    return U * s[None, :]


_ORIG_TRUNCATE = M.truncate
_ORIG_SPECTRUM = M.spectrum
_ORIG_COMP = M.compensation
_ORIG_BACKWARD = M.backward
_ORIG_COMPRESS = M.compress
_ORIG_MARGIN = M.margin
_ORIG_EXACT = M.exact_backward

MUTATIONS = [
    ("truncate", _truncate_strict),
    ("truncate", _truncate_off_by_one),
    ("truncate", _truncate_no_oversampling),
    ("truncate", _truncate_energy_not_squared),
    ("spectrum", _spectrum_ascending),
    ("spectrum", _spectrum_unsorted_vectors),
    ("compensation", _comp_wrong_sign),
    ("compensation", _comp_uses_E),
    ("backward", _backward_swaps_pq),
    ("backward", _backward_last_sample_only),
    ("backward", _backward_gx_without_expand_transpose),
    ("backward", _backward_gx_sign),
    ("compress", _compress_reversed_tokens),
    ("Accumulator", _AccPerChannel),
    ("flops_lowrank_formula", _lowrank_formula_wrong),
    ("eps_as_f32", _eps_unrounded),
    ("margin", _margin_shift_up),
    ("margin", _margin_shift_down),
    ("margin", _margin_absolute),
    ("exact_backward", _exact_gx_scaled),
    ("exact_backward", _exact_gw_first_sample),
    ("canonical_signs", _signs_untouched),
    ("canonical_signs", _signs_tie_to_last),
    ("canonical_signs", _signs_largest_value),
]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f.__name__ for _, f in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(M, name, fn)
    monkeypatch.setattr(O, name, fn)
    assert _fails(pins.ALL_CHECKS), f"no pin caught the planted mistake {fn.__name__}"


def test_unmutated_oracle_passes_all():
    assert not _fails(pins.ALL_CHECKS)
