"""CPU oracle for the memory-efficient Swish activation -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``libmeswish`` and
the ``memory_efficient_activation_amd`` binding) never imports, links or runs
it, and it imports nothing from the product path.

The arithmetic lives in ``swish_oracle.c`` (plain C, binary64, compiled with
gcc into ``liboracle.so``); this module only marshals numpy arrays in and out.

What it computes (cited by page title and section):

* [P1] "Memory efficient Swish", "What is a Swish activation function?" and
  "How is Swish implemented?": y = x * Sigmoid(alpha x), Sigmoid(t) = 1/(1+e^-t).
* [P1] "How is the memory efficient version Swish implemented?": backward from
  the input alone, dx = dy * s * (1 + t (1 - s)), t = alpha x, s = Sigmoid(t)
  (alpha other than 1 by the product rule; the page prints alpha = 1).
* Results are rounded once, to nearest even, to binary32 or bfloat16.
* [P3] "What activations cost, in memory and in arithmetic", Given: the
  activation family ReLU, LeakyReLU, sigmoid, tanh, GELU (erf) and GELU
  (tanh approximation), each with its textbook derivative.

Every function here is pinned by ``tests/test_oracle_pins.py`` against facts
that do not come from the oracle itself (closed forms, finite differences,
PyTorch fp64 autograd of the naive module, library sigmoid, exact rational
rounding, the worked numbers of page 3).  No function is "parity unpinned";
infinite inputs give the limits as x -> +-inf, pinned by their closed forms.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "swish_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

F32 = 0
BF16 = 1

# Activation codes of the oracle's family (its own numbering).
ACTS = {"swish": 0, "relu": 1, "leaky_relu": 2, "sigmoid": 3, "tanh": 4,
        "gelu_erf": 5, "gelu_tanh": 6}

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (no HIP, no fast-math) and return the path."""
    cmd = ["gcc", *GCC_FLAGS, source, "-o", output, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return output


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    c_size, c_void = ctypes.c_size_t, ctypes.c_void_p
    lib.oracle_round_f32.argtypes = [ctypes.c_double]
    lib.oracle_round_f32.restype = ctypes.c_float
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_round_n.argtypes = [ctypes.c_int, c_void, c_void, c_size]
    lib.oracle_round_n.restype = None
    lib.oracle_sigmoid.argtypes = [ctypes.c_double]
    lib.oracle_sigmoid.restype = ctypes.c_double
    lib.oracle_swish_fwd.argtypes = [ctypes.c_int, c_void, c_void, c_size,
                                     ctypes.c_float, ctypes.c_int]
    lib.oracle_swish_fwd.restype = ctypes.c_int
    lib.oracle_swish_bwd.argtypes = [ctypes.c_int, c_void, c_void, c_void, c_void,
                                     c_size, ctypes.c_float, ctypes.c_int]
    lib.oracle_swish_bwd.restype = ctypes.c_int
    lib.oracle_swish_fwd_f64.argtypes = [ctypes.c_double, ctypes.c_double]
    lib.oracle_swish_fwd_f64.restype = ctypes.c_double
    lib.oracle_swish_bwd_f64.argtypes = [ctypes.c_double, ctypes.c_double,
                                         ctypes.c_double,
                                         ctypes.POINTER(ctypes.c_double)]
    lib.oracle_swish_bwd_f64.restype = ctypes.c_double
    lib.oracle_act_f64.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double]
    lib.oracle_act_f64.restype = ctypes.c_double
    lib.oracle_act_grad_f64.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_double, ctypes.POINTER(ctypes.c_double)]
    lib.oracle_act_grad_f64.restype = ctypes.c_double
    lib.oracle_act_fwd.argtypes = [ctypes.c_int, ctypes.c_int, c_void, c_void, c_size,
                                   ctypes.c_float, ctypes.c_int]
    lib.oracle_act_fwd.restype = ctypes.c_int
    lib.oracle_act_bwd.argtypes = [ctypes.c_int, ctypes.c_int, c_void, c_void, c_void, c_void,
                                   c_size, ctypes.c_float, ctypes.c_int]
    lib.oracle_act_bwd.restype = ctypes.c_int
    return lib


_LIB = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load liboracle.so (building it first if it is missing)."""
    global _LIB
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _LIB is None:
        if not os.path.exists(LIBRARY):
            build()
        _LIB = _declare(ctypes.CDLL(LIBRARY))
    return _LIB


class Oracle:
    """numpy front end over one loaded copy of the oracle library."""

    def __init__(self, lib: ctypes.CDLL | None = None):
        self.lib = lib if lib is not None else load()

    # --- element-wise binary64 values (unrounded) ---------------------
    def swish_f64(self, x: float, alpha: float) -> float:
        return self.lib.oracle_swish_fwd_f64(float(x), float(alpha))

    def grad_f64(self, x: float, dy: float, alpha: float) -> tuple[float, float]:
        m = ctypes.c_double()
        g = self.lib.oracle_swish_bwd_f64(float(x), float(dy), float(alpha),
                                          ctypes.byref(m))
        return g, m.value

    def sigmoid_f64(self, t: float) -> float:
        return self.lib.oracle_sigmoid(float(t))

    # --- rounding ------------------------------------------------------
    def round_f32(self, v: float) -> np.float32:
        return np.float32(self.lib.oracle_round_f32(float(v)))

    def round_bf16(self, v: float) -> int:
        return int(self.lib.oracle_round_bf16(float(v)))

    def round_array(self, v: np.ndarray, dtype: str) -> np.ndarray:
        """Round binary64 values once to "f32" (float32 array) or "bf16"
        (uint16 bit patterns), to nearest even."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, dtype=np.float32 if dtype == "f32" else np.uint16)
        self.lib.oracle_round_n(F32 if dtype == "f32" else BF16, v.ctypes.data, out.ctypes.data,
                                v.size)
        return out

    # --- arrays ----------------------------------------------------------
    @staticmethod
    def _dtype_code(a: np.ndarray) -> int:
        if a.dtype == np.float32:
            return F32
        if a.dtype == np.uint16:
            return BF16
        raise TypeError("oracle arrays are float32 or uint16 (bfloat16 bits), "
                        f"got {a.dtype}")

    def fwd(self, x: np.ndarray, alpha: float, threads: int = 1) -> np.ndarray:
        """Rounded forward over a contiguous array (float32 or bf16 bits)."""
        x = np.ascontiguousarray(x)
        code = self._dtype_code(x)
        y = np.empty_like(x)
        rc = self.lib.oracle_swish_fwd(code, x.ctypes.data, y.ctypes.data, x.size,
                                       float(np.float32(alpha)), int(threads))
        if rc != 0:
            raise RuntimeError(f"oracle_swish_fwd failed ({rc})")
        return y

    def bwd(self, x: np.ndarray, dy: np.ndarray, alpha: float, threads: int = 1,
            want_scale: bool = True) -> tuple[np.ndarray, np.ndarray | None]:
        """Rounded backward and (optionally) the binary64 error scale."""
        x = np.ascontiguousarray(x)
        dy = np.ascontiguousarray(dy)
        if x.shape != dy.shape or x.dtype != dy.dtype:
            raise ValueError("x and dy must have the same shape and dtype")
        code = self._dtype_code(x)
        dx = np.empty_like(x)
        scale = np.empty(x.shape, dtype=np.float64) if want_scale else None
        rc = self.lib.oracle_swish_bwd(code, x.ctypes.data, dy.ctypes.data,
                                       dx.ctypes.data,
                                       scale.ctypes.data if want_scale else None,
                                       x.size, float(np.float32(alpha)), int(threads))
        if rc != 0:
            raise RuntimeError(f"oracle_swish_bwd failed ({rc})")
        return dx, scale

    # --- the activation family ------------------------------------------
    def act_f64(self, act: str, x: float, p: float = 0.0) -> float:
        return self.lib.oracle_act_f64(ACTS[act], float(x), float(p))

    def act_grad_f64(self, act: str, x: float, dy: float, p: float = 0.0) -> tuple[float, float]:
        m = ctypes.c_double()
        g = self.lib.oracle_act_grad_f64(ACTS[act], float(x), float(dy), float(p), ctypes.byref(m))
        return g, m.value

    def act_fwd(self, act: str, x: np.ndarray, p: float = 0.0, threads: int = 1) -> np.ndarray:
        x = np.ascontiguousarray(x)
        code = self._dtype_code(x)
        y = np.empty_like(x)
        rc = self.lib.oracle_act_fwd(ACTS[act], code, x.ctypes.data, y.ctypes.data, x.size,
                                     float(np.float32(p)), int(threads))
        if rc != 0:
            raise RuntimeError(f"oracle_act_fwd failed ({rc})")
        return y

    def act_bwd(self, act: str, x: np.ndarray, dy: np.ndarray, p: float = 0.0, threads: int = 1,
                want_scale: bool = True) -> tuple[np.ndarray, np.ndarray | None]:
        x = np.ascontiguousarray(x)
        dy = np.ascontiguousarray(dy)
        if x.shape != dy.shape or x.dtype != dy.dtype:
            raise ValueError("x and dy must have the same shape and dtype")
        code = self._dtype_code(x)
        dx = np.empty_like(x)
        scale = np.empty(x.shape, dtype=np.float64) if want_scale else None
        rc = self.lib.oracle_act_bwd(ACTS[act], code, x.ctypes.data, dy.ctypes.data,
                                     dx.ctypes.data, scale.ctypes.data if want_scale else None,
                                     x.size, float(np.float32(p)), int(threads))
        if rc != 0:
            raise RuntimeError(f"oracle_act_bwd failed ({rc})")
        return dx, scale

    def fwd_grouped(self, xs, alpha: float, threads: int = 1):
        """The grouped forward is the per-tensor forward applied in turn."""
        return [self.fwd(x, alpha, threads) for x in xs]

    def bwd_grouped(self, xs, dys, alpha: float, threads: int = 1,
                    want_scale: bool = True):
        """The grouped backward is the per-tensor backward applied in turn."""
        return [self.bwd(x, dy, alpha, threads, want_scale) for x, dy in zip(xs, dys)]
