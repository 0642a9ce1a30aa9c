"""memory_efficient_activation_amd -- memory-efficient Swish for MI355X.

The hot path is libmeswish.so (HIP kernels for gfx950 behind a C ABI,
declared in include/meswish.h).  This package is a thin binding over it:

* ``swish_fwd``, ``swish_bwd``, ``swish_fwd_grouped``, ``swish_bwd_grouped``
  -- tensor-level calls with the C ABI's names;
* ``SwishFn`` / ``swish`` / ``MemoryEfficientSwish`` -- autograd function and
  module that keep only the input between forward and backward;
* ``naive.Swish`` -- the plain module, for comparisons;
* ``inputs`` -- seeded synthetic workloads; ``accounting`` -- byte counts.

The shared library is loaded on first use; importing the package does not
need a GPU.
"""

from .functional import copy_bytes, swish_bwd, swish_bwd_grouped, swish_fwd, swish_fwd_grouped
from .module import MemoryEfficientSwish, SwishFn, swish
from ._lib import MeswishError

__all__ = [
    "swish_fwd", "swish_bwd", "swish_fwd_grouped", "swish_bwd_grouped", "copy_bytes",
    "SwishFn", "swish", "MemoryEfficientSwish", "MeswishError",
]
