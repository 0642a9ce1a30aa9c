"""memory_efficient_activation_amd -- memory-efficient Swish for MI355X.

The hot path is libmeswish.so (HIP kernels for gfx950 behind a C ABI,
declared in include/meswish.h and include/dense_bn.h).  This package is a thin binding over it:

* ``swish_fwd``, ``swish_bwd``, ``swish_fwd_grouped``, ``swish_bwd_grouped``
  -- tensor-level calls with the C ABI's names;
* ``SwishFn`` / ``swish`` / ``MemoryEfficientSwish`` -- autograd function and
  module that keep only the input between forward and backward;
* ``act_fwd`` / ``act_bwd`` / ``ActFn`` / ``MemoryEfficientActivation`` -- the
  same scheme for ReLU, LeakyReLU, sigmoid, tanh and both GELUs;
* ``dense`` -- the shared-buffer DenseNet layer stage (concatenation +
  batch normalization + ReLU written to a shared buffer and recomputed in
  the backward; include/dense_bn.h) and its bottleneck modules;
* ``naive.Swish`` -- the plain module, for comparisons;
* ``inputs`` -- seeded synthetic workloads; ``accounting`` -- byte counts.

The shared library is loaded on first use; importing the package does not
need a GPU.
"""

from .functional import (act_bwd, act_fwd, copy_bytes, swish_bwd, swish_bwd_grouped, swish_fwd,
                         swish_fwd_grouped)
from .module import ActFn, MemoryEfficientActivation, MemoryEfficientSwish, SwishFn, swish
from ._lib import MeswishError
from . import dense

__all__ = [
    "swish_fwd", "swish_bwd", "swish_fwd_grouped", "swish_bwd_grouped", "copy_bytes",
    "act_fwd", "act_bwd", "ActFn", "MemoryEfficientActivation",
    "SwishFn", "swish", "MemoryEfficientSwish", "MeswishError",
]
