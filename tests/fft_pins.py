"""Pins of the FFT-convolution oracle (oracle/fft_oracle.py).

Each ``pin_*`` takes the oracle module ``o`` and raises AssertionError when
it disagrees with a fact that does not come from the oracle itself:

* the 2-D DFT written out as a double sum of complex exponentials (brute
  force on small maps), Hermitian symmetry, Parseval's identity, the shift
  theorem, and the round trip through the inverse;
* binary64 PyTorch CPU conv2d (cross-correlation) and its autograd for the
  input and weight gradients -- an independent implementation of (1)-(3);
* the convolution theorem, on which the method rests: the spectral path
  equals the direct definition for all three operations;
* special kernels: a unit impulse (the output is a crop of the input), a
  kernel as large as the map (one dot product), 1 x 1 kernels (a matrix
  product per pixel).
"""

from __future__ import annotations

import numpy as np


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed, S=2, F=3, G=4, n=8, k=3):
    r = _rng(seed)
    x = r.standard_normal((S, F, n, n))
    w = r.standard_normal((G, F, k, k))
    g = r.standard_normal((S, G, n - k + 1, n - k + 1))
    return x, w, g


def pin_dft_by_definition(o):
    for seed, n, m in ((1, 4, 4), (2, 8, 5), (3, 8, 8), (4, 16, 3)):
        x = _rng(seed).standard_normal((2, m, m))
        xp = np.zeros((2, n, n))
        xp[:, :m, :m] = x
        X = o.rfft2_half(x, n)
        assert X.shape == (2, n, n // 2 + 1)
        p = np.arange(n)
        for u in range(n):
            for v in range(n // 2 + 1):
                e = np.exp(-2j * np.pi * (u * p[:, None] + v * p[None, :]) / n)
                want = (xp * e).sum(axis=(-2, -1))
                assert np.allclose(X[:, u, v], want, rtol=1e-12, atol=1e-12 * np.abs(x).sum())


def pin_parseval_and_symmetry(o):
    n = 16
    x = _rng(5).standard_normal((3, n, n))
    X = o.rfft2_half(x, n)
    # Full spectrum from the half: X(u, v) = conj(X(-u, -v)).
    full = np.zeros((3, n, n), complex)
    full[:, :, :n // 2 + 1] = X
    for v in range(n // 2 + 1, n):
        full[:, :, v] = np.conj(X[:, (-np.arange(n)) % n, n - v])
    assert np.allclose((np.abs(full) ** 2).sum(axis=(1, 2)) / n ** 2,
                       (x ** 2).sum(axis=(1, 2)), rtol=1e-12)
    # Columns v = 0 and n/2 are Hermitian along u on their own.
    for v in (0, n // 2):
        assert np.allclose(X[:, :, v], np.conj(X[:, (-np.arange(n)) % n, v]), atol=1e-10)
    assert np.allclose(X[:, 0, 0], x.sum(axis=(1, 2)), rtol=1e-13)


def pin_shift_theorem_and_round_trip(o):
    n = 8
    x = _rng(6).standard_normal((2, n, n))
    X = o.rfft2_half(x, n)
    dy, dx = 3, 5
    Xs = o.rfft2_half(np.roll(x, (dy, dx), axis=(1, 2)), n)
    u = np.arange(n)[:, None]
    v = np.arange(n // 2 + 1)[None, :]
    assert np.allclose(Xs, X * np.exp(-2j * np.pi * (u * dy + v * dx) / n), atol=1e-11)
    assert np.allclose(o.irfft2_crop(X, n, n), x, atol=1e-13)
    assert np.allclose(o.irfft2_crop(X, n, 5), x[:, :5, :5], atol=1e-13)


def pin_torch_conv2d(o):
    import torch
    import torch.nn.functional as F
    for seed, S, Fi, G, n, k in ((7, 2, 3, 4, 8, 3), (8, 1, 2, 2, 9, 4), (9, 3, 1, 2, 6, 6),
                                 (10, 2, 2, 3, 7, 1)):
        x, w, g = _case(seed, S, Fi, G, n, k)
        tx = torch.tensor(x, requires_grad=True)
        tw = torch.tensor(w, requires_grad=True)
        ty = F.conv2d(tx, tw)
        ty.backward(torch.tensor(g))
        assert np.allclose(o.fprop_direct(x, w), ty.detach().numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(o.bprop_direct(g, w, n), tx.grad.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(o.accgrad_direct(x, g, k), tw.grad.numpy(), rtol=1e-12, atol=1e-11)


def pin_convolution_theorem(o):
    for seed, n, k in ((11, 8, 3), (12, 16, 5), (13, 8, 8), (14, 16, 1)):
        x, w, g = _case(seed, 2, 3, 2, n, k)
        sc = o.fprop_scale(x, w)[:, :, None, None]
        assert np.all(np.abs(o.fprop_fft(x, w) - o.fprop_direct(x, w)) <= 1e-12 * sc)
        sc = o.bprop_scale(g, w)[:, :, None, None]
        assert np.all(np.abs(o.bprop_fft(g, w, n) - o.bprop_direct(g, w, n)) <= 1e-12 * sc)
        sc = o.accgrad_scale(x, g)[:, :, None, None]
        assert np.all(np.abs(o.accgrad_fft(x, g, k) - o.accgrad_direct(x, g, k)) <= 1e-12 * sc)


def pin_special_kernels(o):
    x, w, g = _case(15, 2, 3, 4, 8, 3)
    # Unit impulse at (1, 2) on input feature 1 -> output = shifted crop.
    d = np.zeros((4, 3, 3, 3))
    d[:, 1, 1, 2] = 1.0
    y = o.fprop_direct(x, d)
    assert np.array_equal(y, np.broadcast_to(x[:, 1:2, 1:7, 2:8], y.shape))
    # Kernel as large as the map: one dot product per (s, f').
    wk = _rng(16).standard_normal((4, 3, 8, 8))
    assert np.allclose(o.fprop_direct(x, wk)[:, :, 0, 0],
                       np.einsum("sfij,gfij->sg", x, wk), rtol=1e-13)
    # 1 x 1 kernels: a matrix product per pixel.
    w1 = _rng(17).standard_normal((4, 3, 1, 1))
    assert np.allclose(o.fprop_direct(x, w1), np.einsum("gf,sfij->sgij", w1[:, :, 0, 0], x),
                       rtol=1e-13)
    # Scales bound every element (Cauchy-Schwarz).
    assert np.all(np.abs(o.fprop_direct(x, w)) <= o.fprop_scale(x, w)[:, :, None, None] + 1e-12)


def pin_scales_attained(o):
    """Each error scale is the Cauchy-Schwarz bound of its output elements
    and is attained where that bound is sharp, so it is tight and not merely
    an upper bound (an inflated scale would loosen every tolerance built on
    it).  The cases have kernels as large as the maps, so each operation
    reduces to dot products written out here with einsum:
      forward: x[s, f] a positive multiple of w[g0, f]   -> y = sum ||x|| ||w||;
      input gradient: every w[g, f] one spike at the same place, with the
        sign of g[s0, g]                                 -> the spike's gradient;
      weight gradient: every x[s, f] one spike, with the sign of g[s, g0];
      spectrum: a constant map, all of whose energy is in the zero bin
        (Parseval: the bin's magnitude is n ||x||)."""
    r = _rng(71)
    S, F, G, n = 3, 4, 5, 6
    # Forward.
    w = r.standard_normal((G, F, n, n))
    g0 = 2
    x = r.uniform(0.5, 2.0, (S, F))[:, :, None, None] * w[g0][None]
    y = np.einsum("sfij,gfij->sg", x, w)
    sc = o.fprop_scale(x, w)
    assert np.allclose(sc[:, g0], np.abs(y[:, g0]), rtol=1e-12, atol=0), (sc[:, g0], y[:, g0])
    assert np.all(np.abs(y) <= sc * (1 + 1e-12))
    # Input gradient: the output gradient is 1 x 1 (m = 1).
    g = r.standard_normal((S, G, 1, 1))
    s0, i0, j0 = 1, 4, 2
    w = np.zeros((G, F, n, n))
    w[:, :, i0, j0] = np.sign(g[s0, :, 0, 0])[:, None] * r.uniform(0.5, 2.0, (G, F))
    gx = np.einsum("sg,gfij->sfij", g[:, :, 0, 0], w)
    sc = o.bprop_scale(g, w)
    assert np.allclose(sc[s0], np.abs(gx[s0, :, i0, j0]), rtol=1e-12, atol=0)
    assert np.all(np.abs(gx) <= sc[:, :, None, None] * (1 + 1e-12))
    # Weight gradient.
    x = np.zeros((S, F, n, n))
    x[:, :, i0, j0] = np.sign(g[:, g0, 0, 0])[:, None] * r.uniform(0.5, 2.0, (S, F))
    gw = np.einsum("sfij,sg->gfij", x, g[:, :, 0, 0])
    sc = o.accgrad_scale(x, g)
    assert np.allclose(sc[g0], np.abs(gw[g0, :, i0, j0]), rtol=1e-12, atol=0)
    assert np.all(np.abs(gw) <= sc[:, :, None, None] * (1 + 1e-12))
    # Spectrum of a constant map.
    c = np.full((2, n, n), -1.75)
    X = np.fft.fft2(c)
    sc = o.spectrum_scale(c, n)
    assert np.allclose(sc, np.abs(X[:, 0, 0]), rtol=1e-12, atol=0), (sc, X[:, 0, 0])
    assert np.all(np.abs(X) <= sc[:, None, None] * (1 + 1e-12))


ALL_PINS = [pin_dft_by_definition, pin_parseval_and_symmetry, pin_shift_theorem_and_round_trip,
            pin_torch_conv2d, pin_convolution_theorem, pin_special_kernels,
            pin_scales_attained]
