"""Parity rules between a result and the oracle -- TEST INFRASTRUCTURE.

* binary32 forward: |g - o| <= rtol * max(|o|, 2^-126)           (rtol = 1e-5)
* binary32 backward: |g - o| <= rtol * max(m, 2^-126), where m is the oracle's
  error scale |dy| s (1 + |t| (1 - s)) -- the size of the terms of the sum,
  which is what any evaluation's rounding error is proportional to; it equals
  |o| wherever t >= 0 and differs from it only near the zero of Swish'.
* bfloat16: the bit patterns, mapped to ordered integers (negative patterns
  to -(bits & 0x7FFF), so both zeros map to 0), differ by at most 1.
* NaN must meet NaN and nothing else; the two zeros compare equal.

* bfloat16 with a term scale (results that sum terms of either sign, such as
  batch normalization's): ordered distance at most 1 from the oracle's
  rounded value, or |g - v| <= rtol * m with v the oracle's binary64 value --
  an evaluation in binary32 arithmetic may move a cancelled result by more
  than one bfloat16 step of its own size, but not by more than rtol times
  the size of its terms.

The floor 2^-126 (the smallest binary32 normal) reads "relative error" for
references that are zero or subnormal, where a relative measure is
undefined.  o is the oracle's value rounded to the output type.

Every report counts the elements that break the rule (n_bad, NaN mismatches
included) and gives the index of the first one in the input arrays
(first_bad, -1 if none).  tests/compare_pins.py pins these rules on
hand-built cases at both sides of each bound, and tests/test_compare_cpu.py
checks that planted mistakes in this file are caught.
"""

from __future__ import annotations

import numpy as np

FLOOR = np.float64(2.0 ** -126)


def ord_bf16(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _nan_mask(got: np.ndarray, want: np.ndarray, is_nan):
    return is_nan(got), is_nan(want)


def bf16_report(got: np.ndarray, want: np.ndarray) -> dict:
    got = np.asarray(got, dtype=np.uint16).ravel()
    want = np.asarray(want, dtype=np.uint16).ravel()
    isn = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
    gn, wn = _nan_mask(got, want, isn)
    ok = ~(gn | wn)
    d = np.abs(ord_bf16(got[ok]) - ord_bf16(want[ok]))
    bad_mask = np.zeros(got.size, dtype=bool)
    bad_mask[np.nonzero(ok)[0]] = d > 1
    bad_mask |= gn != wn
    bad = int(np.count_nonzero(bad_mask))
    return {"n": int(got.size), "max_ulp": int(d.max()) if d.size else 0,
            "n_off_by_one": int(np.count_nonzero(d == 1)), "n_bad": bad, "ok": bad == 0,
            "first_bad": int(np.nonzero(bad_mask)[0][0]) if bad else -1}


def f32_report(got: np.ndarray, want: np.ndarray, scale: np.ndarray | None = None,
               rtol: float = 1e-5) -> dict:
    """Forward rule if scale is None, else the backward rule with scale m."""
    got = np.asarray(got, dtype=np.float32).ravel().astype(np.float64)
    want = np.asarray(want, dtype=np.float32).ravel().astype(np.float64)
    gn, wn = _nan_mask(got, want, np.isnan)
    ok = ~(gn | wn)
    ref = np.abs(want[ok]) if scale is None else np.asarray(scale, np.float64).ravel()[ok]
    den = np.maximum(ref, FLOOR)
    with np.errstate(invalid="ignore"):
        err = np.abs(got[ok] - want[ok]) / den
    err = np.where(got[ok] == want[ok], 0.0, err)  # equal infinities
    bad_mask = np.zeros(got.size, dtype=bool)
    bad_mask[np.nonzero(ok)[0]] = ~(err <= rtol)
    bad_mask |= gn != wn
    bad = int(np.count_nonzero(bad_mask))
    return {"n": int(got.size), "max_rel": float(err.max()) if err.size else 0.0,
            "n_bad": bad, "ok": bad == 0,
            "first_bad": int(np.nonzero(bad_mask)[0][0]) if bad else -1}


def bf16_scaled_report(got: np.ndarray, want_bits: np.ndarray, want64: np.ndarray,
                       scale: np.ndarray, rtol: float = 1e-5) -> dict:
    """bfloat16 rule with a term scale m (see the module docstring)."""
    got = np.asarray(got, dtype=np.uint16).ravel()
    want_bits = np.asarray(want_bits, dtype=np.uint16).ravel()
    want64 = np.asarray(want64, np.float64).ravel()
    scale = np.asarray(scale, np.float64).ravel()
    isn = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
    gn, wn = _nan_mask(got, want_bits, isn)
    ok = ~(gn | wn)
    d = np.abs(ord_bf16(got[ok]) - ord_bf16(want_bits[ok]))
    gv = (got[ok].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    near = np.abs(gv - want64[ok]) <= rtol * np.maximum(scale[ok], FLOOR)
    bad_mask = np.zeros(got.size, dtype=bool)
    bad_mask[np.nonzero(ok)[0]] = (d > 1) & ~near
    bad_mask |= gn != wn
    bad = int(np.count_nonzero(bad_mask))
    return {"n": int(got.size), "max_ulp": int(d.max()) if d.size else 0,
            "n_off_by_one": int(np.count_nonzero(d == 1)),
            "n_beyond_one_within_scale": int(np.count_nonzero((d > 1) & near)),
            "n_bad": bad, "ok": bad == 0,
            "first_bad": int(np.nonzero(bad_mask)[0][0]) if bad else -1}
