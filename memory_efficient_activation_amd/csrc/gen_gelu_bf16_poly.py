"""Coefficients of the short Gaussian-tail polynomials used by GELU (erf)
with bfloat16 I/O in act_math.h.

With binary32 I/O the kernels evaluate the tail h(a) = erfc(a / sqrt 2) / 2
= Phi(-a) (a = |x|) through Numerical Recipes' erfcc form,
t exp(-z^2 + Q(t)) with t = 1 / (1 + z / 2): a reciprocal, a degree-9
polynomial and an exponential.  bfloat16 results need far less, so for them
h is one exponential of one polynomial: h(a) = 2^L(s), where L is the
Chebyshev interpolant (values at the Chebyshev nodes) of the exact
log2 h(a) on the fast path's range a in [0, 6] (x >= -6; beyond a = 6 the
clamped value is below every binary32 ulp of 1 - h), in the variable
s = a / 3 - 1 in [-1, 1], converted to monomial form.

* degree 6 for the forward: relative error of h below 5e-5, far inside half
  a bfloat16 ulp (2^-9);
* degree 9 for the backward: Phi + x phi cancels near x = -0.752, and the
  bfloat16 inputs nearest that zero need h to about 1e-5; degree 9 gives
  1.5e-6.

The script prints the binary32 coefficients (highest power first, the
order of the Horner loop) and the largest relative error of h when the
polynomial is evaluated in binary32 on a fine grid.

    python memory_efficient_activation_amd/csrc/gen_gelu_bf16_poly.py
"""

import mpmath
import numpy as np

A_MAX = 6.0
mpmath.mp.dps = 40


def log2_tail(a: float) -> float:
    return float(mpmath.log(mpmath.erfc(mpmath.mpf(a) / mpmath.sqrt(2)) / 2, 2))


def fit(degree: int):
    k = np.arange(degree + 1)
    s_nodes = np.cos((2 * k + 1) * np.pi / (2 * (degree + 1)))
    vals = [log2_tail(3.0 * (s + 1.0)) for s in s_nodes]
    cheb = np.polynomial.chebyshev.Chebyshev.fit(s_nodes, vals, degree, domain=[-1.0, 1.0])
    mono = cheb.convert(kind=np.polynomial.Polynomial).coef  # ascending powers of s
    c32 = [np.float32(c) for c in mono]
    worst = 0.0
    for a in np.linspace(0.0, A_MAX, 6001):
        s = np.float32(np.float32(a) * np.float32(1.0 / 3.0) - np.float32(1.0))
        p = c32[-1]
        for c in reversed(c32[:-1]):
            p = np.float32(np.float32(p * s) + c)
        h32 = 2.0 ** float(p)
        h = float(mpmath.erfc(mpmath.mpf(float(np.float32(a))) / mpmath.sqrt(2)) / 2)
        worst = max(worst, abs(h32 / h - 1.0))
    return c32, worst


if __name__ == "__main__":
    for degree in (6, 9):
        c32, worst = fit(degree)
        print(f"degree {degree}, highest power first:")
        print(", ".join(np.format_float_positional(c, unique=True) + "f" for c in reversed(c32)))
        print(f"max relative error of h evaluated in binary32 on [0, {A_MAX}]: {worst:.3e}")
