"""The parity rules of oracle/compare.py against hand-built cases, and
planted mistakes in the rules that those cases must catch (CPU only).

A mutant is the comparator's source with one textual change (a loosened
bound, a dropped NaN check, a wrong ordering of bfloat16 patterns, a
misaligned scale), executed as a fresh module; at least one pin of
``compare_pins.py`` must fail on it.
"""

import os
import types

import numpy as np
import pytest

import compare_pins
from oracle import compare

SOURCE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "oracle", "compare.py")


@pytest.mark.parametrize("pin", compare_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(compare)


NAN_CHECK = "    bad_mask |= gn != wn\n"
IS_NAN = "isn = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)"

# name: (text in compare.py, replacement, which occurrence of the text)
MUTANTS = {
    "bf16_two_steps": ("] = d > 1\n", "] = d > 2\n", 0),
    "bf16_distance_signed": ("d = np.abs(ord_bf16(got[ok]) - ord_bf16(want[ok]))",
                             "d = ord_bf16(got[ok]) - ord_bf16(want[ok])", 0),
    "bf16_drops_nan_check": (NAN_CHECK, "", 0),
    "bf16_inf_counts_as_nan": (IS_NAN, "isn = lambda b: ((b & 0x7F80) == 0x7F80)", 0),
    "ord_drops_sign": ("np.where(b & 0x8000, -(b & 0x7FFF), b)", "np.where(b & 0x8000, (b & 0x7FFF), b)", 0),
    "ord_negative_zero_apart": ("np.where(b & 0x8000, -(b & 0x7FFF), b)",
                                "np.where(b & 0x8000, -(b & 0x7FFF) - 1, b)", 0),
    "f32_tenfold_bound": ("~(err <= rtol)", "~(err <= 10 * rtol)", 0),
    "f32_bound_at_2e5": ("~(err <= rtol)", "~(err <= 2 * rtol)", 0),
    "f32_drops_nan_check": (NAN_CHECK, "", 1),
    "f32_nan_passes": ("gn, wn = _nan_mask(got, want, np.isnan)",
                       "gn, wn = _nan_mask(got, want, np.isnan); wn = gn", 0),
    "floor_loosened": ("FLOOR = np.float64(2.0 ** -126)", "FLOOR = np.float64(2.0 ** -100)", 0),
    "floor_dropped": ("den = np.maximum(ref, FLOOR)", "den = ref", 0),
    "scale_ignored": ("ref = np.abs(want[ok]) if scale is None else np.asarray(scale, np.float64).ravel()[ok]",
                      "ref = np.abs(want[ok])", 0),
    "scale_doubled": ("ref = np.abs(want[ok]) if scale is None else np.asarray(scale, np.float64).ravel()[ok]",
                      "ref = np.abs(want[ok]) if scale is None else 2 * np.asarray(scale, np.float64).ravel()[ok]", 0),
    "scale_misaligned": ("np.asarray(scale, np.float64).ravel()[ok]",
                         "np.asarray(scale, np.float64).ravel()[:int(ok.sum())]", 0),
    "equal_infinities_unhandled": ("err = np.where(got[ok] == want[ok], 0.0, err)  # equal infinities",
                                   "err = err", 0),
    "first_bad_last": ('"first_bad": int(np.nonzero(bad_mask)[0][0]) if bad else -1}',
                       '"first_bad": int(np.nonzero(bad_mask)[0][-1]) if bad else -1}', 0),
    "scaled_loosened": ("near = np.abs(gv - want64[ok]) <= rtol * np.maximum(scale[ok], FLOOR)",
                        "near = np.abs(gv - want64[ok]) <= 10 * rtol * np.maximum(scale[ok], FLOOR)", 0),
    "scaled_against_rounded": ("near = np.abs(gv - want64[ok])",
                               "near = np.abs(gv - (want_bits[ok].astype(np.uint32) << 16)"
                               ".view(np.float32).astype(np.float64))", 0),
    "scaled_two_steps": ("(d > 1) & ~near", "(d > 2) & ~near", 0),
    "scaled_drops_nan_check": (NAN_CHECK, "", 2),
    "scaled_inf_counts_as_nan": (IS_NAN, "isn = lambda b: ((b & 0x7F80) == 0x7F80)", 1),
}


def _replace_nth(src, old, new, k):
    at = -1
    for _ in range(k + 1):
        at = src.find(old, at + 1)
        assert at >= 0, (old, k)
    return src[:at] + new + src[at + len(old):]


def _mutant(name):
    old, new, k = MUTANTS[name]
    src = open(SOURCE).read()
    mod = types.ModuleType(f"compare_{name}")
    exec(compile(_replace_nth(src, old, new, k), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def test_mutation_sites_exist():
    src = open(SOURCE).read()
    assert src.count(NAN_CHECK) == 3 and src.count(IS_NAN) == 2
    for name, (old, _, k) in MUTANTS.items():
        assert src.count(old) > k, name


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in compare_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
