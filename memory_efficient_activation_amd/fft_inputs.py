"""Seeded synthetic inputs for the FFT convolution layer.

Like ``inputs``, this module holds no arithmetic of the method: it draws
random numbers (numpy ``Generator(PCG64(seed))``) in binary64 and converts
them to binary32.  The oracle and the GPU path receive exactly these bits.

"Fast Training of Convolutional Networks through FFTs" (the algorithm and
GPU sections) analyses layers of f input and f' output feature maps of
n x n pixels, k x k kernels and minibatches of S; its table of typical
sizes is lost in extraction.  The measured layer here is one such layer:
S = 128, f = 96, f' = 256, n = 32, k = 7 (n' = 26) -- the minibatch and
feature counts of a second convolution stage of an ImageNet-era network on
32 x 32 maps.  Inputs x ~ N(0, 1), kernels w ~ N(0, 1 / (f k^2)) (unit
output variance), output gradients g ~ N(0, 1); drawn in that order from
one generator.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BENCH_LAYER = {"S": 128, "f": 96, "fo": 256, "n": 32, "k": 7}


@dataclass
class ConvLayer:
    name: str
    S: int
    f: int
    fo: int
    n: int
    k: int
    x: np.ndarray      # float32 [S, f, n, n]
    w: np.ndarray      # float32 [fo, f, k, k]
    g: np.ndarray      # float32 [S, fo, n', n']

    @property
    def m(self) -> int:
        return self.n - self.k + 1


def conv_layer(S: int, f: int, fo: int, n: int, k: int, seed: int = 0, name: str = "") -> ConvLayer:
    rng = np.random.default_rng(seed)
    m = n - k + 1
    x = rng.standard_normal((S, f, n, n)).astype(np.float32)
    w = (rng.standard_normal((fo, f, k, k)) / np.sqrt(f * k * k)).astype(np.float32)
    g = rng.standard_normal((S, fo, m, m)).astype(np.float32)
    return ConvLayer(name or f"conv S={S} f={f} f'={fo} n={n} k={k}", S, f, fo, n, k, x, w, g)


def bench_layer(seed: int = 0) -> ConvLayer:
    b = BENCH_LAYER
    return conv_layer(b["S"], b["f"], b["fo"], b["n"], b["k"], seed,
                      name=f"S={b['S']} f={b['f']} f'={b['fo']} n={b['n']} k={b['k']}")
