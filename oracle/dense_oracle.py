"""CPU oracle for the shared-buffer DenseNet layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the GPU path.

What it computes (README of efficient_densenet_pytorch, "A memory-efficient
implementation of DenseNets", section Motivation): the input of a DenseNet
layer is the concatenation of all earlier feature maps along the channel
axis; batch normalization and then ReLU are applied to it, and these
intermediate maps are what the efficient implementation keeps only in
shared memory and recomputes in the backward pass.  The layer stage is

    u = concat_j(x_j)                      x_j: [N, C_j, P], u: [N, C, P]
    mean_c = mean over (n, p) of u[:, c, :]
    var_c  = mean over (n, p) of (u - mean_c)^2     (batch statistics)
    xhat   = (u - mean_c) / sqrt(var_c + eps)
    h      = gamma_c xhat + beta_c
    z      = max(h, 0)

with the textbook training-mode batch normalization (statistics of the
batch, biased variance, eps inside the square root) -- the pages name batch
normalization without restating it.  Its backward, for an upstream gradient
dz of z, with M = N P values per channel:

    g      = dz where h > 0, else 0
    dbeta  = sum over (n, p) of g
    dgamma = sum over (n, p) of g xhat
    du     = gamma / sqrt(var + eps) (g - dbeta / M - xhat dgamma / M)

and du is split back into one gradient per source feature map.

Everything is evaluated in binary64 with numpy and rounded once, to nearest
even, to the output type by the C oracle's pinned rounding routine.  Each
function returns, beside its values, the size of the terms that its result
sums (the error scale m of the tolerance rule), for the same reason as the
Swish oracle does.

Pinned by ``tests/test_dense_oracle.py``: binary64 PyTorch CPU autograd of
torch.cat + batch_norm + relu, closed forms (constant channels, two-value
channels), invariants of the backward, finite differences, channel
independence of the concatenation, and planted mistakes.
"""

from __future__ import annotations

import numpy as np


def concat(sources):
    """u = concatenation of the sources along the channel axis."""
    return np.concatenate([np.asarray(s, np.float64) for s in sources], axis=1)


def batch_stats(u):
    """Per-channel mean and biased variance over batch and positions."""
    mean = u.mean(axis=(0, 2))
    var = ((u - mean[None, :, None]) ** 2).mean(axis=(0, 2))
    return mean, var


def forward(sources, gamma, beta, eps):
    """z = ReLU(gamma xhat + beta) of the concatenated sources, in binary64.

    Returns (z, aux) where aux holds mean, var, xhat, h and the error scale
    of z where h > 0: |gamma| r (|u| + |mean|) + |beta|, the size of the
    terms gamma r u, gamma r mean and beta that h sums (r = 1/sqrt(var + eps))."""
    u = concat(sources)
    gamma = np.asarray(gamma, np.float64)[None, :, None]
    beta = np.asarray(beta, np.float64)[None, :, None]
    mean, var = batch_stats(u)
    xhat = (u - mean[None, :, None]) / np.sqrt(var + eps)[None, :, None]
    h = gamma * xhat + beta
    z = np.maximum(h, 0.0)
    r = (1.0 / np.sqrt(var + eps))[None, :, None]
    terms = np.abs(gamma) * r * (np.abs(u) + np.abs(mean)[None, :, None]) + np.abs(beta)
    scale = np.where(h > 0, terms, 0.0)
    return z, {"mean": mean, "var": var, "xhat": xhat, "h": h, "scale": scale}


def split(u, channels):
    """Cut a [N, C, P] array back into the sources' channel blocks."""
    out, c0 = [], 0
    for c in channels:
        out.append(u[:, c0:c0 + c, :])
        c0 += c
    return out


def backward(sources, dz, gamma, beta, eps):
    """Gradients of the sources, gamma and beta for the upstream gradient
    dz of z, recomputing everything from the sources.

    Returns (dsources, dgamma, dbeta, aux); aux holds the error scales:
    for du, |gamma| r (|g| + |dbeta| / M + (|u| + |mean|) r |dgamma| / M);
    for dgamma, sum |g| (|u| + |mean|) r; for dbeta, sum |g| -- the sizes of
    the terms each result sums, xhat counted as its two terms u r and
    mean r."""
    _, f = forward(sources, gamma, beta, eps)
    dz = np.asarray(dz, np.float64)
    n, c, p = dz.shape
    m = n * p
    g = np.where(f["h"] > 0, dz, 0.0)
    xhat = f["xhat"]
    dbeta = g.sum(axis=(0, 2))
    dgamma = (g * xhat).sum(axis=(0, 2))
    gam = np.asarray(gamma, np.float64)
    r = 1.0 / np.sqrt(f["var"] + eps)
    k = (gam * r)[None, :, None]
    du = k * (g - dbeta[None, :, None] / m - xhat * dgamma[None, :, None] / m)
    xsize = (np.abs(concat(sources)) + np.abs(f["mean"])[None, :, None]) * r[None, :, None]
    du_scale = np.abs(k) * (np.abs(g) + np.abs(dbeta)[None, :, None] / m
                            + xsize * np.abs(dgamma)[None, :, None] / m)
    channels = [np.shape(s)[1] for s in sources]
    aux = {"du_scale": split(du_scale, channels),
           "dgamma_scale": (np.abs(g) * xsize).sum(axis=(0, 2)),
           "dbeta_scale": np.abs(g).sum(axis=(0, 2)),
           "mean": f["mean"], "var": f["var"], "h": f["h"]}
    return split(du, channels), dgamma, dbeta, aux
