"""CPU oracle for FFT-based convolution layers -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the GPU path.

What it computes ("Fast Training of Convolutional Networks through FFTs",
sections on backpropagation, the convolution theorem and the algorithm): a
convolution layer with input maps x[s, f] (n x n, s over the minibatch of
size S, f over the input features), kernels w[f', f] (k x k) and outputs
y[s, f'] of size n' x n', n' = n - k + 1, performs three operations:

    (1) forward         y[s, f']  = sum_f  x[s, f] (*) w[f', f]
    (2) input gradient  gx[s, f]  = sum_f' g[s, f'] (x) w[f', f]
    (3) weight gradient gw[f', f] = sum_s  x[s, f] (*) g[s, f']

with g = dL/dy.  The page's equations are lost in extraction; the reading
taken here is the standard layer of convolutional networks: (*) is the
"valid" cross-correlation, (x) the "full" convolution -- exactly the
operations that make (2) and (3) the gradients of (1).  Written out:

    y[s,f',i,j]  = sum_{f,a,b}  x[s,f,i+a,j+b] w[f',f,a,b]
    gx[s,f,p,q]  = sum_{f',a,b} g[s,f',p-a,q-b] w[f',f,a,b]   (g = 0 outside)
    gw[f',f,a,b] = sum_{s,i,j}  x[s,f,i+a,j+b] g[s,f',i,j]

The FFT method evaluates each of them by the convolution theorem on n x n
circular transforms (no wrap-around reaches the kept outputs, since
n' + k - 1 = n):

    (1) Y = sum_f X conj(W_pad),   y = crop_{n'}(IFFT(Y))
    (2) GX = sum_f' G_pad W_pad,   gx = IFFT(GX)
    (3) GW = sum_s X conj(G_pad),  gw = crop_k(IFFT(GW))

with FFT the 2-D DFT X(u, v) = sum_{p,q} x(p, q) e^{-2 pi i (u p + v q) / n},
zero-padding at the top-left, and only the half spectrum v in [0, n/2]
kept, since the inputs are real (the page's "symmetry properties of FFTs
of real inputs").

The direct functions are the definitions above written as loops over the
kernel offsets (a, b) with numpy sums over the feature axes; the spectral
functions use numpy's FFT (a library primitive) in binary64.  Pinned by
tests/test_fft_oracle.py: the DFT written out as a double sum, Parseval,
the shift theorem, PyTorch CPU binary64 conv2d and its autograd, the
convolution theorem (spectral path = direct path), special kernels, and
planted mistakes.
"""

from __future__ import annotations

import numpy as np


def pad(x, n):
    """Zero-pad the last two axes of x to n x n, data at the top-left."""
    x = np.asarray(x, np.float64)
    m0, m1 = x.shape[-2], x.shape[-1]
    out = np.zeros(x.shape[:-2] + (n, n))
    out[..., :m0, :m1] = x
    return out


def rfft2_half(x, n):
    """Half spectrum [..., n, n // 2 + 1] of each map, zero-padded to n x n."""
    return np.fft.rfft2(pad(x, n), axes=(-2, -1))


def irfft2_crop(spec, n, m):
    """Real n x n maps from half spectra, cropped to the top-left m x m."""
    return np.fft.irfft2(np.asarray(spec, np.complex128), s=(n, n), axes=(-2, -1))[..., :m, :m]


# --- the three operations, direct -----------------------------------------

def fprop_direct(x, w):
    """y[s,f',i,j] = sum_{f,a,b} x[s,f,i+a,j+b] w[f',f,a,b] (valid)."""
    x, w = np.asarray(x, np.float64), np.asarray(w, np.float64)
    n, k = x.shape[-1], w.shape[-1]
    m = n - k + 1
    y = np.zeros((x.shape[0], w.shape[0], m, m))
    for a in range(k):
        for b in range(k):
            y += np.einsum("sfij,gf->sgij", x[:, :, a:a + m, b:b + m], w[:, :, a, b])
    return y


def bprop_direct(g, w, n):
    """gx[s,f,p,q] = sum_{f',a,b} g[s,f',p-a,q-b] w[f',f,a,b] (full)."""
    g, w = np.asarray(g, np.float64), np.asarray(w, np.float64)
    k = w.shape[-1]
    m = g.shape[-1]
    gx = np.zeros((g.shape[0], w.shape[1], n, n))
    for a in range(k):
        for b in range(k):
            gx[:, :, a:a + m, b:b + m] += np.einsum("sgij,gf->sfij", g, w[:, :, a, b])
    return gx


def accgrad_direct(x, g, k):
    """gw[f',f,a,b] = sum_{s,i,j} x[s,f,i+a,j+b] g[s,f',i,j]."""
    x, g = np.asarray(x, np.float64), np.asarray(g, np.float64)
    m = g.shape[-1]
    gw = np.zeros((g.shape[1], x.shape[1], k, k))
    for a in range(k):
        for b in range(k):
            gw[:, :, a, b] = np.einsum("sfij,sgij->gf", x[:, :, a:a + m, b:b + m], g)
    return gw


# --- the frequency-domain stage (per-bin contractions) ---------------------

def freq_fprop(X, W):
    """Y[s,f'] = sum_f X[s,f] conj(W[f',f]), per frequency bin."""
    return np.einsum("sfuv,gfuv->sguv", X, np.conj(W))


def freq_bprop(G, W):
    """GX[s,f] = sum_f' G[s,f'] W[f',f], per frequency bin."""
    return np.einsum("sguv,gfuv->sfuv", G, W)


def freq_accgrad(X, G):
    """GW[f',f] = sum_s X[s,f] conj(G[s,f']), per frequency bin."""
    return np.einsum("sfuv,sguv->gfuv", X, np.conj(G))


# --- the three operations through the convolution theorem ------------------

def fprop_fft(x, w):
    n, k = np.shape(x)[-1], np.shape(w)[-1]
    return irfft2_crop(freq_fprop(rfft2_half(x, n), rfft2_half(w, n)), n, n - k + 1)


def bprop_fft(g, w, n):
    return irfft2_crop(freq_bprop(rfft2_half(g, n), rfft2_half(w, n)), n, n)


def accgrad_fft(x, g, k):
    n = np.shape(x)[-1]
    return irfft2_crop(freq_accgrad(rfft2_half(x, n), rfft2_half(g, n)), n, k)


# --- error scales -----------------------------------------------------------
# Any element of sum_f x_f (*) w_f is at most sum_f ||x_f||_2 ||w_f||_2 in
# magnitude (Cauchy-Schwarz on each window), and an evaluation through
# transforms makes errors proportional to those norms, not to the element:
# the scales below are that bound, one per output map.

def _norms(a):
    return np.sqrt((np.asarray(a, np.float64) ** 2).sum(axis=(-2, -1)))


def fprop_scale(x, w):
    """[S, F'] = sum_f ||x[s,f]|| ||w[f',f]||."""
    return _norms(x) @ _norms(w).T


def bprop_scale(g, w):
    """[S, F] = sum_f' ||g[s,f']|| ||w[f',f]||."""
    return _norms(g) @ _norms(w)


def accgrad_scale(x, g):
    """[F', F] = sum_s ||g[s,f']|| ||x[s,f]||."""
    return _norms(g).T @ _norms(x)


def spectrum_scale(x, n):
    """Per map: the 2-norm of its n x n transform, n ||x||_2 (Parseval)."""
    return n * _norms(x)
