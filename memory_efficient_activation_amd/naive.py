"""The plain Swish module: the baseline the method is measured against.

This module reproduces on purpose the plain module that the blog post
"Memory efficient Swish" lists under "How is Swish implemented?" (a
constructor taking alpha, default 1.0, and a forward returning the input
times the sigmoid of alpha times the input, in eager PyTorch ops).  The
listing's behaviour is what is being compared: autograd keeps its
intermediate feature maps for the backward ("Why simple Swish
implementation is inefficient?"), and the memory-efficient module must give
the same gradients while keeping one map.  It is used only as that
baseline -- by the tests (autograd equivalence, retained bytes) and by the
memory experiment's naive leg -- and is never a fallback of the library.
"""

from __future__ import annotations

import torch
from torch import nn


class Swish(nn.Module):
    def __init__(self, alpha: float = 1.0):
        super().__init__()
        self.alpha = float(alpha)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return x * torch.sigmoid(self.alpha * x)
