"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only draws random numbers
(numpy ``Generator(PCG64(seed))``) and encodes them as binary32 or bfloat16
bit patterns.  The oracle and the GPU path both receive exactly these bits.

Workloads (shapes from the activations the pages size and measure):

1. ``[65536]`` binary32, alpha 1.0; x = 3 * N(0,1) from seed 0, dy = N(0,1)
   from seed 1 -- a small case the oracle finishes instantly.
2. EfficientNet stem activation ``[64, 32, 112, 112]`` NCHW binary32,
   alpha 1.0; x, dy ~ N(0,1) from seeds 0 and 1.  Stands in for the
   EfficientNet feature maps whose memory the blog post measures ("How much
   GPU memory is saved?"), which needs no model weights or data.
3. The transformer-scale tensor of "What activations cost, in memory and in
   arithmetic" (Given; Step 1): ``[8, 2048, 4096]`` = 67,108,864 elements,
   bfloat16 I/O, alpha 1.0; x ~ N(0,1) from seed 0, dy ~ 0.01 N(0,1) from
   seed 1.
4. The same shape in binary32 with alpha 1.5; x is a mixture drawn from seed 0
   in this order: z = standard_normal(n); m = random(n) < 0.01;
   mag = uniform(20, 90, n); sgn = where(random(n) < 0.5, -1, 1);
   x = where(m, sgn * mag, z).  About 1 % of the elements sit in +-[20, 90],
   far enough out to drive e^(-|alpha x|) below the binary32 normal range.
   dy ~ N(0,1) from seed 1.
5. Seven bfloat16 NHWC tensors at batch 32 with the expansion widths of an
   EfficientNet's inverted-bottleneck blocks: 112^2 x 96, 56^2 x 144,
   28^2 x 240, 14^2 x 480, 14^2 x 672, 7^2 x 1152, 7^2 x 1280; tensor i draws
   x ~ N(0,1) and then dy ~ N(0,1) from ``default_rng(i)``.

Values are drawn in binary64, converted to binary32 with ``astype`` (round to
nearest even) and, for bfloat16, from binary32 to bfloat16 by round to
nearest even on the bit pattern.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

EFFICIENTNET_MBCONV_SHAPES = [
    (32, 112, 112, 96),
    (32, 56, 56, 144),
    (32, 28, 28, 240),
    (32, 14, 14, 480),
    (32, 14, 14, 672),
    (32, 7, 7, 1152),
    (32, 7, 7, 1280),
]


@dataclass
class Workload:
    """One synthetic workload: a list of (x, dy) host arrays and alpha."""

    index: int
    name: str
    dtype: str                      # "f32" or "bf16"
    alpha: float
    shapes: list = field(default_factory=list)
    xs: list = field(default_factory=list)      # float32 or uint16 arrays
    dys: list = field(default_factory=list)

    @property
    def numel(self) -> int:
        return int(sum(int(np.prod(s)) for s in self.shapes))


# --------------------------------------------------------------------------
# Encodings (bit-level, no method arithmetic).
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns, round to nearest even.

    NaN stays NaN (quiet).  Used only to encode inputs.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> binary32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def encode(a64: np.ndarray, dtype: str) -> np.ndarray:
    a32 = np.asarray(a64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return a32
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(f"unknown dtype {dtype!r}")


def decode(a: np.ndarray) -> np.ndarray:
    """Host array in either encoding -> binary32 values."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)


# --------------------------------------------------------------------------
# The five workloads.
# --------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "swish fp32 [65536] alpha=1.0",
    2: "swish fp32 NCHW [64,32,112,112] alpha=1.0 (EfficientNet stem)",
    3: "swish bf16 [8,2048,4096] alpha=1.0 (transformer-scale tensor)",
    4: "swish fp32 [8,2048,4096] alpha=1.5 (1% outliers in +-[20,90])",
    5: "swish bf16 grouped, 7 NHWC MBConv tensors at batch 32, alpha=1.0",
}

CONFIG_SHAPES = {
    1: [(65536,)],
    2: [(64, 32, 112, 112)],
    3: [(8, 2048, 4096)],
    4: [(8, 2048, 4096)],
    5: EFFICIENTNET_MBCONV_SHAPES,
}

CONFIG_DTYPES = {1: "f32", 2: "f32", 3: "bf16", 4: "f32", 5: "bf16"}
CONFIG_ALPHAS = {1: 1.0, 2: 1.0, 3: 1.0, 4: 1.5, 5: 1.0}


def _outlier_mixture(rng: np.random.Generator, n: int) -> np.ndarray:
    z = rng.standard_normal(n)
    m = rng.random(n) < 0.01
    mag = rng.uniform(20.0, 90.0, n)
    sgn = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    return np.where(m, sgn * mag, z)


def make(index: int, n: int | None = None) -> Workload:
    """Build workload ``index`` (1..5).

    ``n`` (configs 1-4 only) replaces the element count while keeping the
    value recipe, for parity runs at sizes the oracle finishes quickly.
    """
    if index not in CONFIG_NAMES:
        raise ValueError(f"unknown workload {index}")
    dtype = CONFIG_DTYPES[index]
    w = Workload(index=index, name=CONFIG_NAMES[index], dtype=dtype,
                 alpha=CONFIG_ALPHAS[index])
    if index == 5:
        if n is not None:
            raise ValueError("workload 5 has fixed shapes")
        for i, shape in enumerate(EFFICIENTNET_MBCONV_SHAPES):
            rng = np.random.default_rng(i)
            size = int(np.prod(shape))
            x = rng.standard_normal(size)
            dy = rng.standard_normal(size)
            w.shapes.append(shape)
            w.xs.append(encode(x, dtype))
            w.dys.append(encode(dy, dtype))
        return w

    shape = CONFIG_SHAPES[index][0] if n is None else (int(n),)
    size = int(np.prod(shape))
    rx = np.random.default_rng(0)
    ry = np.random.default_rng(1)
    if index == 1:
        x = 3.0 * rx.standard_normal(size)
        dy = ry.standard_normal(size)
    elif index in (2,):
        x = rx.standard_normal(size)
        dy = ry.standard_normal(size)
    elif index == 3:
        x = rx.standard_normal(size)
        dy = 0.01 * ry.standard_normal(size)
    else:  # 4
        x = _outlier_mixture(rx, size)
        dy = ry.standard_normal(size)
    w.shapes.append(shape)
    w.xs.append(encode(x, dtype))
    w.dys.append(encode(dy, dtype))
    return w


def exhaustive_bf16_finite() -> np.ndarray:
    """All 65,280 finite bfloat16 bit patterns (both zeros included)."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (b & 0x7F80) != 0x7F80
    return b[finite]


def fp32_pattern_sample(stride: int = 4099) -> np.ndarray:
    """Every ``stride``-th binary32 bit pattern that is finite, as float32."""
    u = np.arange(0, 1 << 32, stride, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    return f[np.isfinite(f)]
