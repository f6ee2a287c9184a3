"""Python binding of the INSTANT low-rank backward library (gfx950 HIP, C ABI).

Argument marshalling only: every step runs in the HIP kernels of ``libinstant.so``.
The functions carry the C names of ``include/instant.h`` and take device tensors
(anything with ``data_ptr()``), raw integer pointers, or ``None`` for NULL. Streams
default to PyTorch's current stream on the current device.

Method: notes "INSTANT: Compressing Gradients and Activations for Resource-Efficient
Training" (papernotes.org, ICLR 2026), sections 整体框架 and 关键设计 1-3.

Importing fails loudly when the built library is missing; there is no fallback.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import sys
import weakref

try:  # bind to the HIP runtime PyTorch has already loaded, if PyTorch is present
    import torch  # noqa: F401
except ImportError:  # pragma: no cover
    torch = None

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libinstant.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()')")

_lib = ctypes.CDLL(LIB_PATH)

# ----------------------------------------------------------------------------- enums

INSTANT_OK, INSTANT_E_ARG, INSTANT_E_SHAPE, INSTANT_E_STATE, INSTANT_E_RANK = 0, 1, 2, 3, 4
INSTANT_E_ENERGY, INSTANT_E_NONFINITE, INSTANT_E_NOCONV, INSTANT_E_HIP = 5, 6, 7, 8
INSTANT_FP32, INSTANT_BF16 = 0, 1
INSTANT_COMP_PAPER, INSTANT_COMP_NONE, INSTANT_COMP_RATIO = 0, 1, 2
INSTANT_SOLVER_JACOBI, INSTANT_SOLVER_SUBSPACE = 0, 1
INSTANT_FINALIZE_NONE, INSTANT_FINALIZE_SYNC, INSTANT_FINALIZE_ASYNC = 0, 1, 2


class instant_config(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("Cx", ctypes.c_int32), ("Cy", ctypes.c_int32),
                ("B_max", ctypes.c_int32), ("R_max", ctypes.c_int32), ("p", ctypes.c_int32),
                ("N_t", ctypes.c_int32), ("eps", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("comp", ctypes.c_int32), ("max_sweeps", ctypes.c_int32), ("solver", ctypes.c_int32),
                ("sub_iters", ctypes.c_int32)]


class instant_info(ctypes.Structure):
    _fields_ = [("kx", ctypes.c_int32), ("ky", ctypes.c_int32), ("Rx", ctypes.c_int32),
                ("Ry", ctypes.c_int32), ("sweeps_x", ctypes.c_int32), ("sweeps_g", ctypes.c_int32),
                ("status", ctypes.c_int32), ("cP", ctypes.c_float), ("cQ", ctypes.c_float),
                ("kept_x", ctypes.c_double), ("kept_g", ctypes.c_double),
                ("n_samples_x", ctypes.c_int64), ("n_samples_g", ctypes.c_int64),
                ("generation", ctypes.c_uint32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_vp = ctypes.c_void_p
_st = ctypes.c_int
_sig = {
    "instant_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(instant_config)]),
    "instant_create": (_st, [ctypes.POINTER(_vp), ctypes.POINTER(instant_config), _vp, _vp]),
    "instant_destroy": (_st, [_vp]),
    "instant_calibrate": (_st, [_vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, _vp]),
    "instant_compress_fwd": (_st, [_vp, _vp, ctypes.c_int32, _vp, _vp]),
    "instant_backward": (_st, [_vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp]),
    "instant_backward_static": (_st, [_vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp]),
    "instant_query": (_st, [_vp, ctypes.POINTER(instant_info)]),
    "instant_set_projections": (_st, [_vp, _vp, ctypes.c_int32, _vp, ctypes.c_int32, _vp]),
    "instant_get_projections": (_st, [_vp, _vp, _vp, _vp, _vp, _vp]),
    "instant_get_statistics": (_st, [_vp, _vp, _vp, _vp]),
    "instant_status_str": (ctypes.c_char_p, [_st]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sig)


class InstantError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        super().__init__(f"{where}: {instant_status_str(status)}" if where else instant_status_str(status))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ----------------------------------------------------------------------------- C names

def instant_status_str(s: int) -> str:
    return _lib.instant_status_str(int(s)).decode()


def instant_workspace_bytes(cfg: instant_config) -> int:
    return int(_lib.instant_workspace_bytes(ctypes.byref(cfg)))


def instant_create(cfg: instant_config, workspace, stream=None):
    """Returns (status, handle)."""
    h = _vp()
    s = _lib.instant_create(ctypes.byref(h), ctypes.byref(cfg), _ptr(workspace), _stream(stream))
    return s, h


def instant_destroy(h) -> int:
    return _lib.instant_destroy(h)


def instant_calibrate(h, x, gy, B: int, finalize, stream=None) -> int:
    """finalize: False / 0 (none), True / 1 (synchronous), "async" / 2 (asynchronous)."""
    mode = INSTANT_FINALIZE_ASYNC if finalize == "async" else int(finalize)
    return _lib.instant_calibrate(h, _ptr(x), _ptr(gy), int(B), mode, _stream(stream))


def instant_compress_fwd(h, x, B: int, xhat, stream=None) -> int:
    return _lib.instant_compress_fwd(h, _ptr(x), int(B), _ptr(xhat), _stream(stream))


def instant_backward(h, xhat, gy, w, B: int, gw, gx, stream=None) -> int:
    return _lib.instant_backward(h, _ptr(xhat), _ptr(gy), _ptr(w), int(B), _ptr(gw), _ptr(gx), _stream(stream))


def instant_backward_static(h, xhat, gy, w, B: int, gw, gx, stream=None) -> int:
    return _lib.instant_backward_static(h, _ptr(xhat), _ptr(gy), _ptr(w), int(B), _ptr(gw), _ptr(gx),
                                        _stream(stream))


INSTANT_STATIC_SCRATCH_BYTES = 64 << 20  # include/instant.h


def instant_query(h):
    """Returns (status, instant_info)."""
    info = instant_info()
    s = _lib.instant_query(h, ctypes.byref(info))
    return s, info


def instant_set_projections(h, P, Rx: int, Q, Ry: int, stream=None) -> int:
    return _lib.instant_set_projections(h, _ptr(P), int(Rx), _ptr(Q), int(Ry), _stream(stream))


def instant_get_projections(h, P, Q, sigma_x, sigma_g, stream=None) -> int:
    return _lib.instant_get_projections(h, _ptr(P), _ptr(Q), _ptr(sigma_x), _ptr(sigma_g), _stream(stream))


def instant_get_statistics(h, C_X, C_G, stream=None) -> int:
    return _lib.instant_get_statistics(h, _ptr(C_X), _ptr(C_G), _stream(stream))


# ----------------------------------------------------------------------------- handle owner

def make_config(L, Cx, Cy, B_max, R_max=64, p=2, N_t=100, eps=0.95, dtype="bf16", comp="paper",
                max_sweeps=30, solver="jacobi", sub_iters=6) -> instant_config:
    dt = {"fp32": INSTANT_FP32, "bf16": INSTANT_BF16}[dtype] if isinstance(dtype, str) else int(dtype)
    cp = {"paper": INSTANT_COMP_PAPER, "none": INSTANT_COMP_NONE, "ratio": INSTANT_COMP_RATIO}[comp] \
        if isinstance(comp, str) else int(comp)
    sv = {"jacobi": INSTANT_SOLVER_JACOBI, "subspace": INSTANT_SOLVER_SUBSPACE}[solver] \
        if isinstance(solver, str) else int(solver)
    return instant_config(int(L), int(Cx), int(Cy), int(B_max), int(min(R_max, L)), int(p), int(N_t),
                          float(eps), dt, cp, int(max_sweeps), sv, int(sub_iters))


# Handles still open. They are closed at interpreter exit by an atexit hook, which runs
# before the interpreter tears down its modules and long before the HIP runtime's own
# teardown at process exit: instant_destroy (an event wait, hipEventDestroy, hipHostFree)
# must not run once that teardown has begun.
_LIVE = weakref.WeakSet()


def close_all() -> None:
    """Close every InstantLayer still open (their workspaces stay with their owners)."""
    for lay in list(_LIVE):
        lay.close()


atexit.register(close_all)


class InstantLayer:
    """Owns one handle and its device workspace (a uint8 tensor on the current device).

    Close it with close() (or use it as a context manager); handles still open at
    interpreter exit are closed by an atexit hook, and a garbage-collected handle is closed
    by __del__ unless the interpreter is already finalizing."""

    def __init__(self, cfg: instant_config, device="cuda", stream=None):
        self.cfg = cfg
        self.h = None
        n = instant_workspace_bytes(cfg)
        if n == 0:
            raise InstantError(INSTANT_E_ARG, "instant_workspace_bytes")
        self.workspace = torch.empty(n + 256, dtype=torch.uint8, device=device)
        base = self.workspace.data_ptr()
        self._ws_ptr = (base + 255) // 256 * 256
        s, h = instant_create(cfg, self._ws_ptr, stream)
        if s != INSTANT_OK:
            raise InstantError(s, "instant_create")
        self.h = h
        _LIVE.add(self)

    def close(self):
        if getattr(self, "h", None):
            instant_destroy(self.h)
            self.h = None
        _LIVE.discard(self)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False

    def __del__(self, _finalizing=sys.is_finalizing):
        # during interpreter finalization the HIP runtime may be going away (and this
        # module's globals may already be cleared): leave the small host handle to the process
        # exit (the atexit hook has closed it already)
        if getattr(self, "h", None) is None or _finalizing():
            return
        self.close()

    def _check(self, s, where):
        if s != INSTANT_OK:
            raise InstantError(s, where)

    def calibrate(self, x, gy, B, finalize=False, stream=None) -> int:
        s = instant_calibrate(self.h, x, gy, B, finalize, stream)
        if s in (INSTANT_E_ARG, INSTANT_E_SHAPE, INSTANT_E_STATE, INSTANT_E_HIP):
            raise InstantError(s, "instant_calibrate")
        return s

    def compress_fwd(self, x, B, xhat, stream=None):
        self._check(instant_compress_fwd(self.h, x, B, xhat, stream), "instant_compress_fwd")

    def backward(self, xhat, gy, w, B, gw, gx, stream=None):
        self._check(instant_backward(self.h, xhat, gy, w, B, gw, gx, stream), "instant_backward")

    def backward_static(self, xhat, gy, w, B, gw, gx, stream=None):
        self._check(instant_backward_static(self.h, xhat, gy, w, B, gw, gx, stream), "instant_backward_static")

    def query(self):
        return instant_query(self.h)

    def set_projections(self, P, Rx, Q, Ry, stream=None):
        self._check(instant_set_projections(self.h, P, Rx, Q, Ry, stream), "instant_set_projections")

    def get_projections(self, P, Q, sigma_x=None, sigma_g=None, stream=None):
        self._check(instant_get_projections(self.h, P, Q, sigma_x, sigma_g, stream), "instant_get_projections")

    def get_statistics(self, C_X, C_G, stream=None):
        self._check(instant_get_statistics(self.h, C_X, C_G, stream), "instant_get_statistics")
