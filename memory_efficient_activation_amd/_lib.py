"""ctypes loader for libmeswish.so (the C ABI declared in include/meswish.h,
include/dense_bn.h and include/fft_conv.h).

Argument marshalling only: every element of every pass is computed by the
HIP kernels inside the library.  There is no CPU fallback -- if the library
is missing or the tensors are not on a HIP device, calls raise.
"""

from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libmeswish.so")

# Status codes and dtypes (mirror include/meswish.h).
OK, EINVAL, EALIAS, EHIP, ETOOMANY, ESCRATCH = 0, 1, 2, 3, 4, 5
F32, BF16 = 0, 1
MAX_GROUP = 64

EXPORTED = ("swish_fwd", "swish_bwd", "swish_fwd_grouped", "swish_bwd_grouped",
            "meswish_act_fwd", "meswish_act_bwd",
            "meswish_strerror", "meswish_version", "meswish_copy", "meswish_plan",
            "dense_bn_workspace_bytes", "dense_bn_stats", "dense_bn_relu_fwd", "dense_bn_relu_bwd",
            "dense_bn_relu_bwd_noalloc",
            "fftconv_buffer_bytes", "fftconv_fprop", "fftconv_bprop", "fftconv_accgrad",
            "fftconv_r2c", "fftconv_c2r", "fftconv_cmul")
DENSE_MAX_SOURCES = 64
DENSE_STATIC_WORKSPACE_BYTES = 4 << 20

# Activation codes (mirror meswish_act) and their default parameters.
ACTS = {"swish": 0, "relu": 1, "leaky_relu": 2, "sigmoid": 3, "tanh": 4, "gelu": 5,
        "gelu_tanh": 6}
DEFAULT_PARAM = {"swish": 1.0, "leaky_relu": 0.01}
PATH_NONE, PATH_VECTOR, PATH_ELEMENT = -1, 0, 1


class FwdDesc(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("n", ctypes.c_size_t)]


class BwdDesc(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("dy", ctypes.c_void_p), ("dx", ctypes.c_void_p),
                ("n", ctypes.c_size_t)]


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("head", ctypes.c_longlong), ("nvec", ctypes.c_longlong),
                ("tail", ctypes.c_longlong), ("tiles", ctypes.c_longlong),
                ("grid", ctypes.c_longlong), ("block", ctypes.c_longlong),
                ("elems_per_vector", ctypes.c_longlong), ("vectors_per_tile", ctypes.c_longlong),
                ("launches", ctypes.c_longlong)]


class DenseSource(ctypes.Structure):
    """dense_bn_source of include/dense_bn.h."""
    _fields_ = [("x", ctypes.c_void_p), ("dx", ctypes.c_void_p), ("stats", ctypes.c_void_p),
                ("channels", ctypes.c_int), ("offset", ctypes.c_int)]


class MeswishError(RuntimeError):
    """A non-zero status returned by libmeswish."""

    def __init__(self, status: int, what: str, message: str):
        super().__init__(f"{what}: {message} (status {status})")
        self.status = status


def _signatures() -> dict:
    """Argument and result types of every exported function."""
    vp, sz, f, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float, ctypes.c_int
    src = ctypes.POINTER(DenseSource)
    sig = {
        "swish_fwd": ([vp, vp, sz, f, i, vp], i),
        "swish_bwd": ([vp, vp, vp, sz, f, i, vp], i),
        "swish_fwd_grouped": ([ctypes.POINTER(FwdDesc), i, f, i, vp], i),
        "swish_bwd_grouped": ([ctypes.POINTER(BwdDesc), i, f, i, vp], i),
        "meswish_strerror": ([i], ctypes.c_char_p),
        "meswish_version": ([], i),
        "meswish_copy": ([vp, vp, sz, vp], i),
        "meswish_act_fwd": ([i, vp, vp, sz, f, i, vp], i),
        "meswish_act_bwd": ([i, vp, vp, vp, sz, f, i, vp], i),
        "meswish_plan": ([vp, vp, vp, sz, f, i, i, ctypes.POINTER(Plan)], i),
        "dense_bn_workspace_bytes": ([sz, sz, sz], sz),
        "dense_bn_stats": ([vp, sz, i, sz, i, vp, vp, sz, vp], i),
        "dense_bn_relu_fwd": ([src, i, sz, sz, i, vp, vp, f, vp, i, vp], i),
        "dense_bn_relu_bwd": ([src, i, sz, sz, i, vp, vp, f, vp, vp, vp, vp, sz, i, vp], i),
        "dense_bn_relu_bwd_noalloc": ([src, i, sz, sz, i, vp, vp, f, vp, vp, vp, i, vp], i),
        "fftconv_buffer_bytes": ([i, i, i, i], sz),
        "fftconv_r2c": ([vp, i, i, i, vp, vp], i),
        "fftconv_c2r": ([vp, i, i, i, f, vp, vp], i),
        "fftconv_cmul": ([i, vp, vp, vp, i, i, i, i, vp], i),
    }
    for name in ("fftconv_fprop", "fftconv_bprop", "fftconv_accgrad"):
        sig[name] = ([vp, vp, vp, i, i, i, i, i, vp, sz, vp], i)
    return sig


def _declare(lib: ctypes.CDLL, names=None) -> ctypes.CDLL:
    """Set argtypes/restype of ``names`` (every exported function by default);
    a missing symbol raises AttributeError."""
    sig = _signatures()
    for name in (sig if names is None else names):
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = sig[name]
    return lib


_LIB = None
_LOCK = threading.Lock()


def library(path: str | None = None, names=None) -> ctypes.CDLL:
    """Load libmeswish.so once (after torch, so that both share one HIP runtime).
    With ``path``, load that build instead (not cached), declaring ``names``
    (every exported function by default)."""
    global _LIB
    if path is not None:
        import torch  # noqa: F401  (the HIP runtime torch loads is the one the library binds to)
        return _declare(ctypes.CDLL(path), names)
    with _LOCK:
        if _LIB is None:
            if not os.path.exists(LIBRARY):
                raise RuntimeError(
                    f"{LIBRARY} is not built; run `python -c 'import __graft_entry__ as g; "
                    "g.build()'` (hipcc --offload-arch=gfx950)")
            import torch  # noqa: F401
            _LIB = _declare(ctypes.CDLL(LIBRARY))
    return _LIB


def check(status: int, what: str) -> None:
    if status != OK:
        msg = library().meswish_strerror(status).decode()
        raise MeswishError(status, what, msg)
