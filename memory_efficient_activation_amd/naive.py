"""The plain Swish module, kept for comparisons only.

Blog post "Memory efficient Swish", "How is Swish implemented?": the input
times the sigmoid of alpha times the input, written with eager PyTorch ops.
Autograd keeps its intermediate feature maps for the backward ("Why simple
Swish implementation is inefficient?").  Tests and the memory comparison use
it as the baseline the memory-efficient module is measured against; it is
not a fallback of the library.
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
