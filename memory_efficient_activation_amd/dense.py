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

import contextlib
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


def _current(device: torch.device):
    """A context that makes `device` current, or nothing if it already is."""
    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


class SharedBuffer:
    """Device memory that every layer reuses (README "A memory-efficient
    implementation of DenseNets", Motivation): the normalized map z of the
    layer being computed, and the reduction workspace of the kernels.  Both
    grow to the largest request and are never shrunk.  Kernels use them in
    stream order, so one SharedBuffer serves one stream at a time."""

    def __init__(self):
        self._storage: torch.Tensor | None = None
        self._ws: torch.Tensor | None = None

    @staticmethod
    def _dev(device) -> torch.device:
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        return dev

    def view(self, shape, dtype, device) -> torch.Tensor:
        numel = 1
        for s in shape:
            numel *= int(s)
        nbytes = numel * torch.empty((), dtype=dtype).element_size()
        dev = self._dev(device)
        st = self._storage
        if st is None or st.numel() < nbytes or st.device != dev:
            self._storage = st = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        return st[:nbytes].view(dtype).view(shape)

    def workspace(self, nbytes: int, device) -> torch.Tensor:
        dev = self._dev(device)
        ws = self._ws
        if ws is None or ws.numel() < nbytes or ws.device != dev:
            self._ws = ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        return ws

    @property
    def nbytes(self) -> int:
        return sum(0 if t is None else t.numel() for t in (self._storage, self._ws))


def workspace(n: int, channels: int, hw: int, device, shared: SharedBuffer | None = None
              ) -> torch.Tensor:
    nbytes = _lib.library().dense_bn_workspace_bytes(n, channels, hw)
    if nbytes == 0:
        raise ValueError(f"sizes out of range: n={n}, channels={channels}, hw={hw}")
    if shared is not None:
        return shared.workspace(nbytes, device)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def bn_stats(x: torch.Tensor, shared: SharedBuffer | None = None) -> torch.Tensor:
    """Per-channel batch mean and biased variance of x [N, C, ...] as a
    float64 tensor [C, 2].  `shared` lends its workspace."""
    x = _as_nchw(x, "x")
    n, c, hw = int(x.shape[0]), int(x.shape[1]), _hw(x)
    code = _dtype_code(x)
    stats = torch.empty((c, 2), dtype=torch.float64, device=x.device)
    ws = workspace(n, c, hw, x.device, shared)
    with _current(x.device):
        st = _lib.library().dense_bn_stats(x.data_ptr(), n, c, hw, code, stats.data_ptr(),
                                           ws.data_ptr(), ws.numel(), _stream(x.device))
    _lib.check(st, "dense_bn_stats")
    return stats


def _params(gamma, beta, channels, device):
    for name, p in (("gamma", gamma), ("beta", beta)):
        if p.dtype != torch.float32 or p.numel() != channels or not p.is_contiguous() or \
                p.device != device:
            raise ValueError(f"{name} must be a contiguous float32 tensor of {channels} values "
                             f"on {device}")


class Prepared:
    """A layer's sources as the C ABI takes them: checked once, with the
    descriptor arrays (at most 64 sources per call) built once and reused by
    the forward, the backward's recomputation and the backward."""

    def __init__(self, xs: Sequence[torch.Tensor], stats: Sequence[torch.Tensor]):
        if len(xs) != len(stats):
            raise ValueError("one statistics tensor per source is required")
        if len(xs) == 0:
            raise ValueError("at least one source is required")
        x0 = xs[0]
        _require_device(x0, "xs[0]")
        if x0.dim() < 2:
            raise ValueError(f"sources must be [N, C, ...], got shape {tuple(x0.shape)}")
        self.code = _dtype_code(x0)
        self.dtype, self.device = x0.dtype, x0.device
        self.n, self.hw, self.spatial = int(x0.shape[0]), _hw(x0), tuple(x0.shape[2:])
        self.channels = []
        self.parts = []
        descs, base = [], 0
        dev_index, dtype, n, spatial = x0.get_device(), x0.dtype, self.n, self.spatial
        f64 = torch.float64
        for j, (x, s) in enumerate(zip(xs, stats)):
            # Lean checks: this runs for every source of every layer.
            shp = x.shape
            if x.dtype is not dtype or x.get_device() != dev_index:
                raise ValueError("all sources must share device and dtype")
            if len(shp) < 2 or shp[0] != n or shp[2:] != spatial:
                raise ValueError(f"source {j} has shape {tuple(shp)}, expected "
                                 f"[{n}, C, {', '.join(map(str, spatial))}]")
            if not x.is_contiguous():
                raise ValueError(f"source {j} must be contiguous")
            c = shp[1]
            if s.dtype is not f64 or s.shape != (c, 2) or not s.is_contiguous() or \
                    s.get_device() != dev_index:
                raise ValueError(f"stats[{j}] must be a contiguous float64 [{c}, 2] tensor on "
                                 f"{self.device}")
            descs.append(_lib.DenseSource(x.data_ptr(), 0, s.data_ptr(), c, base))
            self.channels.append(c)
            base += c
            if len(descs) == _lib.DENSE_MAX_SOURCES or j == len(xs) - 1:
                self.parts.append(((_lib.DenseSource * len(descs))(*descs), len(descs),
                                   sum(d.channels for d in descs)))
                descs = []
        self.total = base
        self.shape = (self.n, self.total, *self.spatial)

    def check_params(self, gamma, beta):
        _params(gamma, beta, self.total, self.device)

    def fwd(self, gamma, beta, eps, z):
        lib, sh = _lib.library(), _stream(self.device)
        with _current(self.device):
            for descs, count, _ in self.parts:
                _lib.check(lib.dense_bn_relu_fwd(descs, count, self.n, self.hw, self.total,
                                                 gamma.data_ptr(), beta.data_ptr(), float(eps),
                                                 z.data_ptr(), self.code, sh),
                           "dense_bn_relu_fwd")

    def bwd(self, gamma, beta, eps, dz, shared: SharedBuffer | None = None):
        """Returns (dxs, dgamma, dbeta); the source gradients are views of one
        allocation."""
        flat = torch.empty(self.n * self.total * self.hw, dtype=self.dtype, device=self.device)
        sizes = [self.n * c * self.hw for c in self.channels]
        dxs = [t.view(self.n, c, *self.spatial) for t, c in zip(flat.split(sizes), self.channels)]
        params = torch.empty(2 * self.total, dtype=torch.float32, device=self.device)
        dgamma, dbeta = params[:self.total], params[self.total:]
        lib, sh = _lib.library(), _stream(self.device)
        with _current(self.device):
            j = 0
            for descs, count, chans in self.parts:
                for k in range(count):
                    descs[k].dx = dxs[j + k].data_ptr()
                j += count
                ws = workspace(self.n, chans, self.hw, self.device, shared)
                _lib.check(lib.dense_bn_relu_bwd(descs, count, self.n, self.hw, self.total,
                                                 gamma.data_ptr(), beta.data_ptr(), float(eps),
                                                 dz.data_ptr(), dgamma.data_ptr(),
                                                 dbeta.data_ptr(), ws.data_ptr(), ws.numel(),
                                                 self.code, sh),
                           "dense_bn_relu_bwd")
        return dxs, dgamma, dbeta


def bn_relu_fwd(xs: Sequence[torch.Tensor], stats: Sequence[torch.Tensor], gamma: torch.Tensor,
                beta: torch.Tensor, eps: float = EPS, out: torch.Tensor | None = None
                ) -> torch.Tensor:
    """z = ReLU(gamma (concat(xs) - mean) / sqrt(var + eps) + beta), written
    into `out` (the shared buffer; [N, sum C_j, ...]) or a new tensor.
    Sources beyond 64 are handled by further calls (channels are
    independent)."""
    prep = Prepared([_as_nchw(x, f"xs[{j}]") for j, x in enumerate(xs)], stats)
    prep.check_params(gamma, beta)
    if out is None:
        out = torch.empty(prep.shape, dtype=prep.dtype, device=prep.device)
    elif tuple(out.shape) != prep.shape or out.dtype != prep.dtype or not out.is_contiguous() \
            or out.device != prep.device:
        raise ValueError(f"out must be a contiguous {prep.dtype} tensor of shape {prep.shape}")
    prep.fwd(gamma, beta, eps, out)
    return out


def bn_relu_bwd(xs: Sequence[torch.Tensor], stats: Sequence[torch.Tensor], gamma: torch.Tensor,
                beta: torch.Tensor, dz: torch.Tensor, eps: float = EPS
                ) -> tuple[list[torch.Tensor], torch.Tensor, torch.Tensor]:
    """Gradients (dxs, dgamma, dbeta) of the stage for the gradient dz of z,
    recomputed from the sources."""
    prep = Prepared([_as_nchw(x, f"xs[{j}]") for j, x in enumerate(xs)], stats)
    prep.check_params(gamma, beta)
    dz = _as_nchw(dz, "dz")
    if dz.dtype != prep.dtype or tuple(dz.shape) != prep.shape or dz.device != prep.device:
        raise ValueError("dz must match the concatenated sources in shape, dtype and device")
    return prep.bwd(gamma, beta, eps, dz)


class DenseBnReluConvFn(torch.autograd.Function):
    """conv1x1(ReLU(BN(concat(sources)))) keeping nothing per layer but
    references to the inputs and the statistics."""

    @staticmethod
    def forward(ctx, shared, eps, gamma, beta, weight, n_src, *rest):
        xs, stats = rest[:n_src], rest[n_src:]
        prep = Prepared(xs, stats)
        prep.check_params(gamma, beta)
        z = shared.view(prep.shape, prep.dtype, prep.device)
        prep.fwd(gamma, beta, eps, z)
        out = F.conv2d(z, weight)
        ctx.shared, ctx.eps, ctx.n_src, ctx.prep = shared, eps, n_src, prep
        ctx.save_for_backward(gamma, beta, weight, *xs, *stats)
        return out

    @staticmethod
    def backward(ctx, dout):
        gamma, beta, weight = ctx.saved_tensors[:3]
        prep, n = ctx.prep, ctx.n_src
        # Re-populate the shared buffer (the method's recomputation), then
        # both gradients of the 1x1 convolution in one call.
        z = ctx.shared.view(prep.shape, prep.dtype, prep.device)
        prep.fwd(gamma, beta, ctx.eps, z)
        dz, dweight, _ = torch.ops.aten.convolution_backward(
            dout.contiguous(), z, weight, None, [1, 1], [0, 0], [1, 1], False, [0, 0], 1,
            [True, True, False])
        del z
        dxs, dgamma, dbeta = prep.bwd(gamma, beta, ctx.eps, dz.contiguous(), ctx.shared)
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
