"""The DenseNet-layer oracle against its pins, and planted mistakes that the
pins must catch (CPU only)."""

import os
import types

import numpy as np
import pytest

import dense_pins
from oracle import dense_oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(os.path.dirname(HERE), "oracle", "dense_oracle.py")


@pytest.mark.parametrize("pin", dense_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(dense_oracle)


# (what is planted, text in the oracle, replacement)
MUTANTS = {
    "unbiased_variance": ("** 2).mean(axis=(0, 2))",
                          "** 2).sum(axis=(0, 2)) / (u.shape[0] * u.shape[2] - 1)"),
    "eps_outside_sqrt": ("xhat = (u - mean[None, :, None]) / np.sqrt(var + eps)[None, :, None]",
                         "xhat = (u - mean[None, :, None]) / (np.sqrt(var) + eps)[None, :, None]"),
    "global_mean": ("mean = u.mean(axis=(0, 2))", "mean = u.mean() + 0 * u.mean(axis=(0, 2))"),
    "stats_over_positions_only": ("mean = u.mean(axis=(0, 2))\n    var = ((u - mean[None, :, None]) ** 2).mean(axis=(0, 2))",
                                  "mean = u[0].mean(axis=1)\n    var = ((u[0] - mean[:, None]) ** 2).mean(axis=1)"),
    "mask_from_xhat": ('g = np.where(f["h"] > 0, dz, 0.0)', 'g = np.where(f["xhat"] > 0, dz, 0.0)'),
    "no_mask": ('g = np.where(f["h"] > 0, dz, 0.0)', 'g = dz + 0.0'),
    "drops_mean_term": ("(g - dbeta[None, :, None] / m - xhat", "(g - xhat"),
    "drops_xhat_term": ("- xhat * dgamma[None, :, None] / m)\n", ")\n"),
    "drops_gamma": ("k = (gam * r)[None, :, None]", "k = r[None, :, None]"),
    "wrong_count": ("m = n * p", "m = p"),
    "dgamma_from_u": ("dgamma = (g * xhat)", "dgamma = (g * concat(sources))"),
    "concat_reversed": ("for s in sources], axis=1)", "for s in sources[::-1]], axis=1)"),
    "split_shifted": ("out.append(u[:, c0:c0 + c, :])", "out.append(np.roll(u, 1, axis=1)[:, c0:c0 + c, :])"),
    "leaky_output": ("z = np.maximum(h, 0.0)", "z = np.maximum(h, 0.0) + 0.01 * np.minimum(h, 0.0)"),
    # Inflated error scales (each would loosen the tolerance it sets).
    "fwd_scale_doubled": ("scale = np.where(h > 0, terms, 0.0)", "scale = np.where(h > 0, 2 * terms, 0.0)"),
    "du_scale_doubled": ("du_scale = np.abs(k) * (", "du_scale = 2 * np.abs(k) * ("),
    "du_scale_drops_mean_term": ("np.abs(g) + np.abs(dbeta)[None, :, None] / m\n",
                                 "np.abs(g)\n"),
    "dgamma_scale_doubled": ('"dgamma_scale": (np.abs(g) * xsize)', '"dgamma_scale": 2 * (np.abs(g) * xsize)'),
    "dbeta_scale_doubled": ('"dbeta_scale": np.abs(g).sum(axis=(0, 2))', '"dbeta_scale": 2 * np.abs(g).sum(axis=(0, 2))'),
    "beta_outside_relu": ("z = np.maximum(h, 0.0)", "z = np.maximum(gamma * xhat, 0.0) + beta"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SOURCE).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"dense_oracle_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in dense_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"


def test_round_array_matches_the_pinned_scalar_routines(oracle):
    """The array rounding the dense oracle uses is the Swish oracle's scalar
    routine (pinned in test_oracle_pins.py) applied element by element."""
    rng = np.random.default_rng(23)
    v = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-45, 39, 2000),
                        [0.0, -0.0, 1.00390625, 1.01171875, -2.5e-39, 3.4e38, np.nan]])
    b = oracle.round_array(v, "bf16")
    assert b.dtype == np.uint16
    assert all(int(b[i]) == oracle.round_bf16(v[i]) for i in range(v.size))
    f = oracle.round_array(v, "f32")
    with np.errstate(over="ignore"):
        assert np.array_equal(f, v.astype(np.float32), equal_nan=True)
