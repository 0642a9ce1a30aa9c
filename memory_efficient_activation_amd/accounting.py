"""Byte accounting for the memory-efficient Swish path.

Conventions (decimal units, as the worked problem "What activations cost, in
memory and in arithmetic" uses them in Step 2: 1 MB = 10^6 B, 1 GB = 10^9 B).

* One activation tensor of n elements occupies ``b * n`` bytes, b = 2 for
  bfloat16 and 4 for binary32 (Step 2).
* Algorithmic HBM traffic of the fused kernels: the forward reads x and writes
  y (``2 b n``); the backward reads x and dy and writes dx (``3 b n``).  The
  same page (Conclusion) notes that an activation reads and writes its tensor
  once each, which is what makes it bandwidth bound.
* Bytes kept alive between forward and backward: the memory-efficient
  function keeps only its input (blog post "Memory efficient Swish", "How is
  the memory efficient version Swish implemented?"), ``b n``; the plain module
  keeps three feature maps -- the input, its sigmoid and the product
  ("Why simple Swish implementation is inefficient?"), ``3 b n``.
"""

from __future__ import annotations

ELEMENT_BYTES = {"f32": 4, "bf16": 2}

# Page-3 counting of floating-point operations per element: sigmoid costs
# about 4 (exp, add, divide); the forward adds the alpha scale and the product
# (6 in all) and the backward recomputes sigmoid and forms 1-s, t(1-s), 1+...,
# s*(...), dy*(...) (10 in all).
FLOPS_PER_ELEMENT = {"fwd": 6, "bwd": 10}


def element_bytes(dtype: str) -> int:
    try:
        return ELEMENT_BYTES[dtype]
    except KeyError:
        raise ValueError(f"unknown dtype {dtype!r}") from None


def tensor_bytes(n: int, dtype: str) -> int:
    return int(n) * element_bytes(dtype)


def fwd_bytes(n: int, dtype: str) -> int:
    """Algorithmic bytes of one forward launch: read x, write y."""
    return 2 * tensor_bytes(n, dtype)


def bwd_bytes(n: int, dtype: str) -> int:
    """Algorithmic bytes of one backward launch: read x and dy, write dx."""
    return 3 * tensor_bytes(n, dtype)


def step_bytes(n: int, dtype: str) -> int:
    """Forward plus backward."""
    return fwd_bytes(n, dtype) + bwd_bytes(n, dtype)


def retained_bytes(n: int, dtype: str, naive: bool = False) -> int:
    """Bytes saved for the backward pass: 1 tensor (x) vs 3 for the naive module."""
    return (3 if naive else 1) * tensor_bytes(n, dtype)


def activation_elements(batch: int, seq: int, width: int) -> int:
    """Elements of one [B, T, d] activation tensor."""
    return int(batch) * int(seq) * int(width)


def stored_across_layers(n: int, dtype: str, layers: int) -> int:
    """Bytes of one stored activation tensor per layer over ``layers`` layers."""
    return int(layers) * tensor_bytes(n, dtype)
