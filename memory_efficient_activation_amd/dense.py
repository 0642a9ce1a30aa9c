"""Shared-buffer DenseNet layer stage on libmeswish (include/dense_bn.h).

README of efficient_densenet_pytorch, "A memory-efficient implementation of
DenseNets", Motivation: the concatenation and batch-normalization outputs of
every DenseNet layer go to memory that all layers share and are recomputed
in the backward pass, which turns the quadratic growth of stored feature
maps into linear growth at the cost of some recomputation.

Here a DenseNet-BC bottleneck's first stage -- concatenate the earlier
feature maps, batch-normalize (batch statistics), ReLU, 1x1 convolution --
is one autograd function that keeps nothing per layer but references to its
inputs (which the network keeps anyway) and the per-channel statistics:

* forward: ``dense_bn_relu_fwd`` writes ReLU(BN(concat)) into a buffer
  shared by every layer (the concatenation itself is never formed), and the
  1x1 convolution reads it;
* backward: the same kernel re-populates the shared buffer, the
  convolution's gradients are taken from it, and ``dense_bn_relu_bwd``
  turns the gradient of the buffer into the gradients of every source,
  gamma and beta.

Per-channel batch statistics depend on one feature map only, so each map's
are computed once (``dense_bn_stats``) when the map is produced and reused
by every later layer that reads it.

Tensor-level functions only check and marshal arguments; every element is
computed by the HIP kernels.  There is no CPU path.  The convolutions are
PyTorch's (MIOpen): they are the model around the method, not part of it.
"""

from __future__ import annotations

from typing import Sequence

import torch
import torch.nn as nn
import torch.nn.functional as F

from . import _lib
from .functional import _dtype_code, _require_device, _stream

EPS = float(torch.tensor(1e-5, dtype=torch.float32))  # binary32, as the kernels use it


def _as_nchw(t: torch.Tensor, name: str) -> torch.Tensor:
    _require_device(t, name)
    if t.dim() < 2:
        raise ValueError(f"{name} must be [N, C, ...], got shape {tuple(t.shape)}")
    return t.contiguous()


def _hw(t: torch.Tensor) -> int:
    hw = 1
    for s in t.shape[2:]:
        hw *= int(s)
    return hw


def workspace(n: int, channels: int, hw: int, device) -> torch.Tensor:
    nbytes = _lib.library().dense_bn_workspace_bytes(n, channels, hw)
    if nbytes == 0:
        raise ValueError(f"sizes out of range: n={n}, channels={channels}, hw={hw}")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def bn_stats(x: torch.Tensor) -> torch.Tensor:
    """Per-channel batch mean and biased variance of x [N, C, ...] as a
    float64 tensor [C, 2]."""
    x = _as_nchw(x, "x")
    n, c, hw = int(x.shape[0]), int(x.shape[1]), _hw(x)
    code = _dtype_code(x)
    stats = torch.empty((c, 2), dtype=torch.float64, device=x.device)
    ws = workspace(n, c, hw, x.device)
    with torch.cuda.device(x.device):
        st = _lib.library().dense_bn_stats(x.data_ptr(), n, c, hw, code, stats.data_ptr(),
                                           ws.data_ptr(), ws.numel(), _stream(x.device))
    _lib.check(st, "dense_bn_stats")
    return stats


def _sources(xs, stats, dxs=None):
    if len(xs) != len(stats):
        raise ValueError("one statistics tensor per source is required")
    if len(xs) == 0:
        raise ValueError("at least one source is required")
    x0 = xs[0]
    n, hw = int(x0.shape[0]), _hw(x0)
    descs, off = [], 0
    for j, (x, s) in enumerate(zip(xs, stats)):
        if x.device != x0.device or x.dtype != x0.dtype:
            raise ValueError("all sources must share device and dtype")
        if int(x.shape[0]) != n or tuple(x.shape[2:]) != tuple(x0.shape[2:]):
            raise ValueError(f"source {j} has shape {tuple(x.shape)}, expected [{n}, C, "
                             f"{', '.join(map(str, x0.shape[2:]))}]")
        if not x.is_contiguous():
            raise ValueError(f"source {j} must be contiguous")
        c = int(x.shape[1])
        if s.dtype != torch.float64 or tuple(s.shape) != (c, 2) or not s.is_contiguous() or \
                s.device != x.device:
            raise ValueError(f"stats[{j}] must be a contiguous float64 [{c}, 2] tensor on "
                             f"{x.device}")
        dxp = 0 if dxs is None else dxs[j].data_ptr()
        descs.append(_lib.DenseSource(x.data_ptr(), dxp, s.data_ptr(), c, off))
        off += c
    if len(descs) > _lib.DENSE_MAX_SOURCES:
        raise ValueError(f"at most {_lib.DENSE_MAX_SOURCES} sources per call")
    return (_lib.DenseSource * len(descs))(*descs), n, hw, off


def _params(gamma, beta, channels, device):
    for name, p in (("gamma", gamma), ("beta", beta)):
        if p.dtype != torch.float32 or p.numel() != channels or not p.is_contiguous() or \
                p.device != device:
            raise ValueError(f"{name} must be a contiguous float32 tensor of {channels} values "
                             f"on {device}")


def bn_relu_fwd(xs: Sequence[torch.Tensor], stats: Sequence[torch.Tensor], gamma: torch.Tensor,
                beta: torch.Tensor, eps: float = EPS, out: torch.Tensor | None = None
                ) -> torch.Tensor:
    """z = ReLU(gamma (concat(xs) - mean) / sqrt(var + eps) + beta), written
    into `out` (the shared buffer; [N, sum C_j, ...]) or a new tensor.
    Sources beyond 64 are handled by further calls (channels are
    independent)."""
    xs = [_as_nchw(x, f"xs[{j}]") for j, x in enumerate(xs)]
    total = sum(int(x.shape[1]) for x in xs)
    x0 = xs[0]
    code = _dtype_code(x0)
    _params(gamma, beta, total, x0.device)
    shape = (int(x0.shape[0]), total, *x0.shape[2:])
    if out is None:
        out = torch.empty(shape, dtype=x0.dtype, device=x0.device)
    elif tuple(out.shape) != shape or out.dtype != x0.dtype or not out.is_contiguous() or \
            out.device != x0.device:
        raise ValueError(f"out must be a contiguous {x0.dtype} tensor of shape {shape}")
    lib = _lib.library()
    base = 0
    with torch.cuda.device(x0.device):
        for lo in range(0, len(xs), _lib.DENSE_MAX_SOURCES):
            part = xs[lo:lo + _lib.DENSE_MAX_SOURCES]
            descs, n, hw, _ = _sources(part, stats[lo:lo + _lib.DENSE_MAX_SOURCES])
            for d in descs:
                d.offset += base
            st = lib.dense_bn_relu_fwd(descs, len(part), n, hw, total, gamma.data_ptr(),
                                       beta.data_ptr(), float(eps), out.data_ptr(), code,
                                       _stream(x0.device))
            _lib.check(st, "dense_bn_relu_fwd")
            base += sum(int(x.shape[1]) for x in part)
    return out


def bn_relu_bwd(xs: Sequence[torch.Tensor], stats: Sequence[torch.Tensor], gamma: torch.Tensor,
                beta: torch.Tensor, dz: torch.Tensor, eps: float = EPS
                ) -> tuple[list[torch.Tensor], torch.Tensor, torch.Tensor]:
    """Gradients (dxs, dgamma, dbeta) of the stage for the gradient dz of z,
    recomputed from the sources."""
    xs = [_as_nchw(x, f"xs[{j}]") for j, x in enumerate(xs)]
    total = sum(int(x.shape[1]) for x in xs)
    x0 = xs[0]
    code = _dtype_code(x0)
    _params(gamma, beta, total, x0.device)
    dz = _as_nchw(dz, "dz")
    if dz.dtype != x0.dtype or tuple(dz.shape) != (int(x0.shape[0]), total, *x0.shape[2:]):
        raise ValueError("dz must match the concatenated sources in shape and dtype")
    dxs = [torch.empty_like(x) for x in xs]
    dgamma = torch.empty(total, dtype=torch.float32, device=x0.device)
    dbeta = torch.empty(total, dtype=torch.float32, device=x0.device)
    lib = _lib.library()
    base = 0
    with torch.cuda.device(x0.device):
        for lo in range(0, len(xs), _lib.DENSE_MAX_SOURCES):
            part = xs[lo:lo + _lib.DENSE_MAX_SOURCES]
            descs, n, hw, chans = _sources(part, stats[lo:lo + _lib.DENSE_MAX_SOURCES],
                                           dxs[lo:lo + _lib.DENSE_MAX_SOURCES])
            for d in descs:
                d.offset += base
            ws = workspace(n, chans, hw, x0.device)
            st = lib.dense_bn_relu_bwd(descs, len(part), n, hw, total, gamma.data_ptr(),
                                       beta.data_ptr(), float(eps), dz.data_ptr(),
                                       dgamma.data_ptr(), dbeta.data_ptr(), ws.data_ptr(),
                                       ws.numel(), code, _stream(x0.device))
            _lib.check(st, "dense_bn_relu_bwd")
            base += chans
    return dxs, dgamma, dbeta


class SharedBuffer:
    """One device allocation that every layer's normalized map reuses
    (README "A memory-efficient implementation of DenseNets", Motivation).
    It grows to the largest request and is never shrunk."""

    def __init__(self):
        self._storage: torch.Tensor | None = None

    def view(self, shape, dtype, device) -> torch.Tensor:
        numel = 1
        for s in shape:
            numel *= int(s)
        nbytes = numel * torch.empty((), dtype=dtype).element_size()
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        st = self._storage
        if st is None or st.numel() < nbytes or st.device != dev:
            self._storage = st = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        return st[:nbytes].view(dtype).view(shape)

    @property
    def nbytes(self) -> int:
        return 0 if self._storage is None else self._storage.numel()


class DenseBnReluConvFn(torch.autograd.Function):
    """conv1x1(ReLU(BN(concat(sources)))) keeping nothing per layer but
    references to the inputs and the statistics."""

    @staticmethod
    def forward(ctx, shared, eps, gamma, beta, weight, n_src, *rest):
        xs, stats = list(rest[:n_src]), list(rest[n_src:])
        total = sum(int(x.shape[1]) for x in xs)
        shape = (int(xs[0].shape[0]), total, *xs[0].shape[2:])
        z = shared.view(shape, xs[0].dtype, xs[0].device)
        bn_relu_fwd(xs, stats, gamma, beta, eps, out=z)
        out = F.conv2d(z, weight)
        ctx.shared, ctx.eps, ctx.n_src = shared, eps, n_src
        ctx.save_for_backward(gamma, beta, weight, *xs, *stats)
        return out

    @staticmethod
    def backward(ctx, dout):
        gamma, beta, weight, *rest = ctx.saved_tensors
        n = ctx.n_src
        xs, stats = rest[:n], rest[n:]
        total = sum(int(x.shape[1]) for x in xs)
        shape = (int(xs[0].shape[0]), total, *xs[0].shape[2:])
        dout = dout.contiguous()
        # Re-populate the shared buffer (the method's recomputation).
        z = ctx.shared.view(shape, xs[0].dtype, xs[0].device)
        bn_relu_fwd(xs, stats, gamma, beta, ctx.eps, out=z)
        dweight = torch.nn.grad.conv2d_weight(z, weight.shape, dout)
        dz = torch.nn.grad.conv2d_input(shape, weight, dout)
        del z
        dxs, dgamma, dbeta = bn_relu_bwd(xs, stats, gamma, beta, dz, ctx.eps)
        return (None, None, dgamma, dbeta, dweight, None, *dxs, *([None] * n))


class EfficientBottleneckStage(nn.Module):
    """BN -> ReLU -> 1x1 conv over the concatenation of the sources, with
    shared buffers and recomputation."""

    def __init__(self, in_channels: int, out_channels: int, shared: SharedBuffer,
                 eps: float = EPS):
        super().__init__()
        self.weight = nn.Parameter(torch.empty(out_channels, in_channels, 1, 1))
        nn.init.kaiming_normal_(self.weight)
        self.gamma = nn.Parameter(torch.ones(in_channels))
        self.beta = nn.Parameter(torch.zeros(in_channels))
        self.shared, self.eps = shared, eps

    def forward(self, xs, stats):
        return DenseBnReluConvFn.apply(self.shared, self.eps, self.gamma, self.beta,
                                       self.weight.to(xs[0].dtype), len(xs), *xs, *stats)


class NaiveBottleneckStage(nn.Module):
    """The plain form: torch.cat -> BatchNorm2d (batch statistics) -> ReLU
    -> 1x1 conv; autograd keeps the concatenation and the ReLU output of
    every layer."""

    def __init__(self, in_channels: int, out_channels: int, eps: float = EPS):
        super().__init__()
        self.weight = nn.Parameter(torch.empty(out_channels, in_channels, 1, 1))
        nn.init.kaiming_normal_(self.weight)
        self.gamma = nn.Parameter(torch.ones(in_channels))
        self.beta = nn.Parameter(torch.zeros(in_channels))
        self.eps = eps

    def forward(self, xs, stats=None):
        u = torch.cat(xs, dim=1)
        h = F.batch_norm(u, None, None, self.gamma.to(u.dtype), self.beta.to(u.dtype),
                         training=True, eps=self.eps)
        return F.conv2d(F.relu(h), self.weight.to(u.dtype))
