"""Coefficients of the short erfc polynomial used by GELU (erf) with
bfloat16 I/O in act_math.h.

The kernels evaluate erfc(z) = t exp(-z^2 + Q(t)), t = 1 / (1 + z/2), the
form of Numerical Recipes' erfcc.  With binary32 I/O, Q is that book's
degree-9 Chebyshev fit (fractional error < 1.2e-7).  bfloat16 results need
only about 2^-12, so for them Q is replaced by the degree-4 polynomial this
script computes: Chebyshev interpolation (values at the 5 Chebyshev nodes)
of the exact Q(t) = ln(erfc(z) / t) + z^2 on the fast path's range
t in [1 / (1 + 3 / sqrt 2), 1] (x >= -6), converted to monomial form.
Its maximal error in Q, i.e. the relative error of erfc, is printed too
(about 7e-5).

    python memory_efficient_activation_amd/csrc/gen_gelu_bf16_poly.py
"""

import mpmath
import numpy as np

DEGREE = 4
mpmath.mp.dps = 40
T_MIN = 1.0 / (1.0 + 3.0 / np.sqrt(2.0))


def exact_q(t: float) -> float:
    z = 2.0 * (1.0 / t - 1.0)
    return float(mpmath.log(mpmath.erfc(z) / t) + z * z)


def fit():
    k = np.arange(DEGREE + 1)
    nodes = np.cos((2 * k + 1) * np.pi / (2 * (DEGREE + 1)))
    tn = T_MIN + (1.0 - T_MIN) * (nodes + 1.0) / 2.0
    cheb = np.polynomial.chebyshev.Chebyshev.fit(tn, [exact_q(t) for t in tn], DEGREE,
                                                 domain=[T_MIN, 1.0])
    mono = cheb.convert(kind=np.polynomial.Polynomial).coef  # ascending powers of t
    ts = np.linspace(T_MIN, 1.0, 2001)
    err = max(abs(np.polynomial.Polynomial(mono)(t) - exact_q(t)) for t in ts)
    return mono, err


if __name__ == "__main__":
    mono, err = fit()
    for i, c in enumerate(mono):
        print(f"c{i} = {np.format_float_positional(np.float32(c))}f")
    print(f"max |Q error| on [{T_MIN:.6f}, 1]: {err:.3e}")
