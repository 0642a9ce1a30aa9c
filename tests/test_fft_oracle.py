"""The FFT-convolution oracle against its pins, and planted mistakes that
the pins must catch (CPU only)."""

import os
import types

import numpy as np
import pytest

import fft_pins
from oracle import fft_oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(os.path.dirname(HERE), "oracle", "fft_oracle.py")


@pytest.mark.parametrize("pin", fft_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(fft_oracle)


MUTANTS = {
    "convolution_not_correlation": (
        'y += np.einsum("sfij,gf->sgij", x[:, :, a:a + m, b:b + m], w[:, :, a, b])',
        'y += np.einsum("sfij,gf->sgij", x[:, :, a:a + m, b:b + m], w[:, :, k - 1 - a, k - 1 - b])'),
    "fprop_no_conj": ('return np.einsum("sfuv,gfuv->sguv", X, np.conj(W))',
                      'return np.einsum("sfuv,gfuv->sguv", X, W)'),
    "accgrad_conj_on_x": ('return np.einsum("sfuv,sguv->gfuv", X, np.conj(G))',
                          'return np.einsum("sfuv,sguv->gfuv", np.conj(X), G)'),
    "bprop_conj": ('return np.einsum("sguv,gfuv->sfuv", G, W)',
                   'return np.einsum("sguv,gfuv->sfuv", G, np.conj(W))'),
    "bprop_correlation": ("gx[:, :, a:a + m, b:b + m] += np.einsum(\"sgij,gf->sfij\", g, w[:, :, a, b])",
                          "gx[:, :, a:a + m, b:b + m] += np.einsum(\"sgij,gf->sfij\", g, w[:, :, k - 1 - a, k - 1 - b])"),
    "accgrad_swapped_offset": ('gw[:, :, a, b] = np.einsum("sfij,sgij->gf", x[:, :, a:a + m, b:b + m], g)',
                               'gw[:, :, b, a] = np.einsum("sfij,sgij->gf", x[:, :, a:a + m, b:b + m], g)'),
    "pad_bottom_right": ("out[..., :m0, :m1] = x", "out[..., n - m0:, n - m1:] = x"),
    "crop_bottom_right": ("axes=(-2, -1))[..., :m, :m]", "axes=(-2, -1))[..., -m:, -m:]"),
    "fprop_first_feature_only": ('y += np.einsum("sfij,gf->sgij", x[:, :, a:a + m, b:b + m], w[:, :, a, b])',
                                 'y += np.einsum("sfij,gf->sgij", x[:, :1, a:a + m, b:b + m], w[:, :1, a, b])'),
    "half_spectrum_too_narrow": ("return np.fft.rfft2(pad(x, n), axes=(-2, -1))",
                                 "return np.fft.rfft2(pad(x, n), axes=(-2, -1))[..., :n // 2]"),
    # Inflated error scales (each would loosen the tolerance it sets).
    "fprop_scale_doubled": ("return _norms(x) @ _norms(w).T", "return 2 * _norms(x) @ _norms(w).T"),
    "bprop_scale_doubled": ("return _norms(g) @ _norms(w)\n", "return 2 * _norms(g) @ _norms(w)\n"),
    "accgrad_scale_doubled": ("return _norms(g).T @ _norms(x)", "return 2 * _norms(g).T @ _norms(x)"),
    "spectrum_scale_doubled": ("return n * _norms(x)", "return 2 * n * _norms(x)"),
    "scale_without_root": ("return np.sqrt((np.asarray(a, np.float64) ** 2).sum(axis=(-2, -1)))",
                           "return (np.asarray(a, np.float64) ** 2).sum(axis=(-2, -1)) / 1e3"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SOURCE).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"fft_oracle_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in fft_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
