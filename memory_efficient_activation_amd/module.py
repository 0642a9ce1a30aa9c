"""Autograd function and module of the memory-efficient Swish.

Blog post "Memory efficient Swish" (adeeplearner.github.io, 2021-05-17):

* "How is the memory efficient version Swish implemented?": one autograd
  function whose forward keeps only its input and whose backward recomputes
  the sigmoid from it, wrapped in a module.
* "How is Swish implemented?": the module carries a slope ``alpha`` (a plain
  float, default 1.0) applied inside the sigmoid.

Both passes run in libmeswish's gfx950 kernels (``functional``); the only
tensor kept between forward and backward is x.
"""

from __future__ import annotations

import torch
from torch import nn

from .functional import act_bwd, act_fwd, swish_bwd, swish_fwd


class SwishFn(torch.autograd.Function):
    """y = x * sigmoid(alpha x); backward from the saved input alone."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, alpha: float = 1.0) -> torch.Tensor:
        y = swish_fwd(x, alpha)
        ctx.save_for_backward(x)
        ctx.alpha = float(alpha)
        return y

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        (x,) = ctx.saved_tensors
        return swish_bwd(x, dy, ctx.alpha), None


def swish(x: torch.Tensor, alpha: float = 1.0) -> torch.Tensor:
    return SwishFn.apply(x, alpha)


class MemoryEfficientSwish(nn.Module):
    """Drop-in Swish module that keeps one tensor (its input) for backward."""

    def __init__(self, alpha: float = 1.0):
        super().__init__()
        self.alpha = float(alpha)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return SwishFn.apply(x, self.alpha)

    def extra_repr(self) -> str:
        return f"alpha={self.alpha}"


class ActFn(torch.autograd.Function):
    """Any activation of the family, keeping only the input for backward."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, kind: str, param: float | None = None) -> torch.Tensor:
        y = act_fwd(kind, x, param)
        ctx.save_for_backward(x)
        ctx.kind = kind
        ctx.param = param
        return y

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        (x,) = ctx.saved_tensors
        return act_bwd(ctx.kind, x, dy, ctx.param), None, None


class MemoryEfficientActivation(nn.Module):
    """Activation module (swish, relu, leaky_relu, sigmoid, tanh, gelu,
    gelu_tanh) that keeps one tensor -- its input -- for the backward."""

    def __init__(self, kind: str, param: float | None = None):
        super().__init__()
        from ._lib import ACTS
        if kind not in ACTS:
            raise ValueError(f"unknown activation {kind!r}; one of {sorted(ACTS)}")
        self.kind = kind
        self.param = param

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return ActFn.apply(x, self.kind, self.param)

    def extra_repr(self) -> str:
        return f"kind={self.kind}, param={self.param}"
