"""Pins of the parity rules in oracle/compare.py, on hand-built cases.

The rules decide every GPU pass or fail, so a loosened rule would turn
every parity claim green and fail nothing.  Each ``pin_*`` takes the
comparator module ``c`` and raises AssertionError when a verdict on a
case built by hand, on either side of a bound, differs from what the rule
as stated gives:

* bfloat16: ordered bit patterns (negative patterns to -(bits & 0x7FFF), so
  +0 and -0 are both 0) at most one step apart; NaN meets NaN only;
* binary32 forward: |g - o| <= 1e-5 max(|o|, 2^-126);
* binary32 backward: |g - o| <= 1e-5 max(m, 2^-126), m the error scale;
* bfloat16 with a term scale: at most one step, or |g - v| <= 1e-5 m.

Cases at 0.99 and 1.01 times a bound sit well clear of the rounding of the
values involved (binary32 spacing near 1 is 1.2e-7 relative, subnormal
spacing 2^-149 exactly); the subnormal cases are integer multiples of 2^-149.
``tests/test_compare_cpu.py`` runs these pins on the real module and on
copies with planted mistakes.
"""

from __future__ import annotations

import numpy as np

ONE = 0x3F80           # bfloat16 1.0
MINUS_ONE = 0xBF80     # bfloat16 -1.0
INF, NINF = 0x7F80, 0xFF80
MAX_FINITE = 0x7F7F
QNAN, QNAN_NEG = 0x7FC0, 0xFFC1
SUB = 2.0 ** -149      # smallest binary32 subnormal


def _u16(*v):
    return np.array(v, dtype=np.uint16)


def _f32(*v):
    return np.array(v, dtype=np.float32)


def _verdict(r, ok, first_bad=None):
    assert r["ok"] is ok, r
    assert (r["n_bad"] == 0) is ok, r
    if first_bad is not None:
        assert r["first_bad"] == first_bad, r


# ---------------------------------------------------------------- bfloat16

def pin_bf16_steps(c):
    _verdict(c.bf16_report(_u16(ONE), _u16(ONE)), True, -1)
    r = c.bf16_report(_u16(ONE, MINUS_ONE), _u16(ONE + 1, MINUS_ONE + 1))
    _verdict(r, True, -1)
    assert r["max_ulp"] == 1 and r["n_off_by_one"] == 2, r
    _verdict(c.bf16_report(_u16(ONE + 2), _u16(ONE)), False, 0)
    _verdict(c.bf16_report(_u16(MINUS_ONE), _u16(MINUS_ONE + 2)), False, 0)
    # Across an exponent boundary: 0x3F7F is the step below 1.0.
    _verdict(c.bf16_report(_u16(0x3F7F), _u16(ONE)), True)
    _verdict(c.bf16_report(_u16(0x3F7E), _u16(ONE)), False)
    # The index of the first offending element, and the count.
    r = c.bf16_report(_u16(ONE, ONE + 3, ONE, ONE + 5), _u16(ONE, ONE, ONE, ONE))
    _verdict(r, False, 1)
    assert r["n_bad"] == 2 and r["max_ulp"] == 5, r


def pin_bf16_zeros(c):
    assert list(c.ord_bf16(_u16(0x0000, 0x8000, 0x0001, 0x8001))) == [0, 0, 1, -1]
    _verdict(c.bf16_report(_u16(0x8000), _u16(0x0000)), True)
    assert c.bf16_report(_u16(0x8000), _u16(0x0000))["max_ulp"] == 0
    _verdict(c.bf16_report(_u16(0x8001), _u16(0x0000)), True)
    _verdict(c.bf16_report(_u16(0x0001), _u16(0x8000)), True)
    # The smallest subnormals of opposite signs are two steps apart.
    _verdict(c.bf16_report(_u16(0x0001), _u16(0x8001)), False, 0)
    _verdict(c.bf16_report(_u16(0x8002), _u16(0x0000)), False, 0)


def pin_bf16_nan_and_inf(c):
    _verdict(c.bf16_report(_u16(QNAN), _u16(QNAN_NEG)), True)
    _verdict(c.bf16_report(_u16(QNAN, ONE), _u16(QNAN, QNAN)), False, 1)
    _verdict(c.bf16_report(_u16(QNAN, QNAN), _u16(QNAN, ONE)), False, 1)
    _verdict(c.bf16_report(_u16(INF), _u16(QNAN)), False, 0)
    _verdict(c.bf16_report(_u16(QNAN), _u16(NINF)), False, 0)
    _verdict(c.bf16_report(_u16(INF, NINF), _u16(INF, NINF)), True)
    # Infinity is the pattern after the largest finite value: one step.
    _verdict(c.bf16_report(_u16(INF), _u16(MAX_FINITE)), True)
    _verdict(c.bf16_report(_u16(INF), _u16(MAX_FINITE - 1)), False)
    _verdict(c.bf16_report(_u16(NINF), _u16(INF)), False)
    # A NaN mismatch after a bad finite element counts both.
    r = c.bf16_report(_u16(ONE + 4, QNAN), _u16(ONE, ONE))
    _verdict(r, False, 0)
    assert r["n_bad"] == 2, r


# ---------------------------------------------------------------- binary32

def pin_f32_forward_bound(c):
    for o in (1.0, -3.5e3, 7.25e-20):
        for sign in (1.0, -1.0):
            near = np.float32(o) * np.float32(1.0 + sign * 0.99e-5)
            far = np.float32(o) * np.float32(1.0 + sign * 1.01e-5)
            _verdict(c.f32_report(_f32(near), _f32(o)), True)
            _verdict(c.f32_report(_f32(far), _f32(o)), False, 0)
    # A zero or subnormal reference: the denominator is 2^-126, so an error
    # of k 2^-149 passes for k <= 83 (83 / 2^23 = 9.89e-6) and fails for 84.
    for o in (0.0, -0.0, 2.0 ** -130, -(2.0 ** -140)):
        _verdict(c.f32_report(_f32(o + 83 * SUB), _f32(o)), True)
        _verdict(c.f32_report(_f32(o - 83 * SUB), _f32(o)), True)
        _verdict(c.f32_report(_f32(o + 84 * SUB), _f32(o)), False, 0)
    # Above the floor the reference's own size counts again: at 2^-125 the
    # spacing is 2^-148, and 83 (84) of those are 9.89e-6 (1.0014e-5) of it.
    o = 2.0 ** -125
    _verdict(c.f32_report(_f32(o + 166 * SUB), _f32(o)), True)
    _verdict(c.f32_report(_f32(o + 168 * SUB), _f32(o)), False)


def pin_f32_backward_scale(c):
    o = np.float32(1e-3)
    near, far = np.float32(o + np.float32(0.99e-5)), np.float32(o + np.float32(1.01e-5))
    _verdict(c.f32_report(_f32(near), _f32(o), np.array([1.0])), True)
    _verdict(c.f32_report(_f32(far), _f32(o), np.array([1.0])), False, 0)
    # Without the scale the same error is 1 % of |o|: the forward rule fails it.
    _verdict(c.f32_report(_f32(near), _f32(o)), False)
    # A scale below the floor is floored at 2^-126.
    _verdict(c.f32_report(_f32(83 * SUB), _f32(0.0), np.array([1e-45])), True)
    _verdict(c.f32_report(_f32(84 * SUB), _f32(0.0), np.array([0.0])), False)
    # The scale of element i goes with element i, also past NaN elements.
    r = c.f32_report(_f32(np.nan, near, far), _f32(np.nan, o, o), np.array([1e-30, 1.0, 2.0]))
    _verdict(r, True)
    r = c.f32_report(_f32(np.nan, near, far), _f32(np.nan, o, o), np.array([1.0, 1.0, 0.5]))
    _verdict(r, False, 2)


def pin_f32_nan_inf_zero(c):
    inf, big = np.float32(np.inf), np.finfo(np.float32).max
    _verdict(c.f32_report(_f32(np.nan), _f32(np.nan)), True)
    _verdict(c.f32_report(_f32(np.nan, 1.0), _f32(np.nan, np.nan)), False, 1)
    _verdict(c.f32_report(_f32(np.nan, np.nan), _f32(np.nan, 1.0)), False, 1)
    _verdict(c.f32_report(_f32(inf, -inf), _f32(inf, -inf)), True)
    _verdict(c.f32_report(_f32(inf, -inf), _f32(inf, -inf), np.array([1.0, 1.0])), True)
    _verdict(c.f32_report(_f32(big), _f32(inf)), False, 0)
    _verdict(c.f32_report(_f32(inf), _f32(big)), False, 0)
    _verdict(c.f32_report(_f32(-inf), _f32(inf)), False, 0)
    _verdict(c.f32_report(_f32(-0.0), _f32(0.0)), True)
    _verdict(c.f32_report(_f32(0.0), _f32(-0.0), np.array([0.0])), True)
    r = c.f32_report(_f32(1.0, 2.0, 3.0), _f32(1.0, 2.5, 3.5))
    _verdict(r, False, 1)
    assert r["n_bad"] == 2, r


# ------------------------------------------------- bfloat16 with a term scale

def pin_bf16_scaled(c):
    # want = 2^-10 exactly (0x3A80); three steps up is 3 2^-17 = 2.29e-5 away.
    want_bits, v64 = _u16(0x3A80), np.array([2.0 ** -10])
    r = c.bf16_scaled_report(_u16(0x3A81), want_bits, v64, np.array([0.0]))
    _verdict(r, True)
    r = c.bf16_scaled_report(_u16(0x3A83), want_bits, v64, np.array([3.0]))   # 3e-5 >= 2.29e-5
    _verdict(r, True)
    assert r["n_beyond_one_within_scale"] == 1, r
    r = c.bf16_scaled_report(_u16(0x3A83), want_bits, v64, np.array([2.0]))   # 2e-5 < 2.29e-5
    _verdict(r, False, 0)
    # The distance to the unrounded value counts, not to the rounded one:
    # v64 one step below want, got two steps above want, so 1.53e-5 from
    # want but 2.29e-5 from v64.
    v = np.array([2.0 ** -10 - 2.0 ** -17])
    _verdict(c.bf16_scaled_report(_u16(0x3A82), want_bits, v, np.array([2.0])), False)
    _verdict(c.bf16_scaled_report(_u16(0x3A82), want_bits, v, np.array([2.4])), True)
    # NaN meets NaN only; scale of element i goes with element i.
    r = c.bf16_scaled_report(_u16(QNAN, 0x3A83), _u16(QNAN, 0x3A80),
                             np.array([np.nan, 2.0 ** -10]), np.array([0.0, 3.0]))
    _verdict(r, True)
    r = c.bf16_scaled_report(_u16(ONE, 0x3A80), _u16(QNAN, 0x3A80),
                             np.array([np.nan, 2.0 ** -10]), np.array([1.0, 1.0]))
    _verdict(r, False, 0)
    r = c.bf16_scaled_report(_u16(0x3A80, QNAN), _u16(0x3A80, 0x3A80),
                             np.array([2.0 ** -10, 2.0 ** -10]), np.array([1e9, 1e9]))
    _verdict(r, False, 1)
    # Infinities are numbers, not NaN.
    r = c.bf16_scaled_report(_u16(INF, NINF), _u16(INF, NINF), np.array([np.inf, -np.inf]),
                             np.array([np.inf, np.inf]))
    _verdict(r, True)
    r = c.bf16_scaled_report(_u16(ONE, INF), _u16(ONE, QNAN), np.array([1.0, np.nan]),
                             np.array([1.0, 1.0]))
    _verdict(r, False, 1)


ALL_PINS = [pin_bf16_steps, pin_bf16_zeros, pin_bf16_nan_and_inf, pin_f32_forward_bound,
            pin_f32_backward_scale, pin_f32_nan_inf_zero, pin_bf16_scaled]
