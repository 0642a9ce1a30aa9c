"""Seeded synthetic inputs for the shared-buffer DenseNet layer.

Like ``inputs``, this module holds no arithmetic of the method: it draws
random numbers (numpy ``Generator(PCG64(seed))``) and encodes them as
binary32 or bfloat16 bit patterns.  The oracle and the GPU path both receive
exactly these bits.

The reference workload is the README of efficient_densenet_pytorch ("A
memory-efficient implementation of DenseNets", section Performance): a
DenseNet-BC with 100 layers at batch 64, on CIFAR-sized 32 x 32 inputs, with
the demo's growth rate 12 (section Usage).  A DenseNet-BC of depth 100 has
three dense blocks of (100 - 4) / 6 = 16 bottleneck layers; the first block
starts from 2 k = 24 channels, and each transition halves the channel count
(compression 0.5) and the resolution.  Layer i of a block sees
c0 + i k channels: the block input plus i earlier layer outputs.

Per-channel statistics differ on purpose, so that the batch statistics are
not all alike: source channel c is offset_c + scale_c N(0, 1) with
offset_c ~ N(0, 1) and scale_c ~ U(0.5, 2).  gamma ~ 1 + 0.25 N(0, 1),
beta ~ 0.5 N(0, 1) (binary32), dz ~ N(0, 1); all from one generator, in
this order: per source (offset, scale, values), then gamma, beta, dz.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .inputs import encode

GROWTH = 12
BATCH = 64
BLOCK_LAYERS = 16
# (block input channels, height = width) of the three dense blocks.
BLOCKS = [(24, 32), (108, 16), (150, 8)]
# batch normalization's eps, as the binary32 value the kernels receive.
EPS = float(np.float32(1e-5))


def block_layer_channels(block: int, layer: int) -> list[int]:
    """Source channel counts seen by layer `layer` (0-based) of dense block
    `block` (0-based): the block input, then one growth-sized map per
    earlier layer."""
    c0, _ = BLOCKS[block]
    return [c0] + [GROWTH] * layer


@dataclass
class DenseLayer:
    name: str
    dtype: str                 # "f32" or "bf16"
    n: int                     # batch
    hw: int                    # positions per channel (H * W)
    channels: list             # C_j of each source
    sources: list              # encoded arrays [n, C_j, hw]
    gamma: np.ndarray          # float32 [C]
    beta: np.ndarray           # float32 [C]
    dz: np.ndarray             # encoded [n, C, hw]
    eps: float = EPS

    @property
    def total_channels(self) -> int:
        return int(sum(self.channels))


def dense_layer(channels, n: int, hw: int, dtype: str, seed: int = 0, eps: float = EPS,
                name: str = "") -> DenseLayer:
    rng = np.random.default_rng(seed)
    sources = []
    for c in channels:
        offset = rng.standard_normal(c)
        scale = rng.uniform(0.5, 2.0, c)
        x = offset[None, :, None] + scale[None, :, None] * rng.standard_normal((n, c, hw))
        sources.append(encode(x, dtype))
    total = int(sum(channels))
    gamma = (1.0 + 0.25 * rng.standard_normal(total)).astype(np.float32)
    beta = (0.5 * rng.standard_normal(total)).astype(np.float32)
    dz = encode(rng.standard_normal((n, total, hw)), dtype)
    return DenseLayer(name or f"dense {list(channels)} n={n} hw={hw} {dtype}", dtype, n, hw,
                      list(channels), sources, gamma, beta, dz, eps)


def densenet_bc100_layer(block: int = 0, layer: int = BLOCK_LAYERS - 1, dtype: str = "f32",
                         n: int = BATCH, seed: int = 0) -> DenseLayer:
    """Layer `layer` of dense block `block` of DenseNet-BC-100 at batch 64."""
    chans = block_layer_channels(block, layer)
    side = BLOCKS[block][1]
    return dense_layer(chans, n, side * side, dtype, seed,
                       name=f"DenseNet-BC-100 block {block + 1} layer {layer + 1}, "
                            f"{sum(chans)} channels, {n}x{side}x{side} {dtype}")
