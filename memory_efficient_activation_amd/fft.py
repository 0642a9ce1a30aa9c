"""FFT convolution layers on libmeswish (include/fft_conv.h).

"Fast Training of Convolutional Networks through FFTs": the forward pass,
the input gradient and the weight gradient of a convolution layer all pair
every f-indexed map with every f'-indexed map, so each map is transformed
once and every pairing becomes a pointwise product in the frequency domain.
The frequency representations live in one buffer that every layer reuses
(the page's memory-saving choice), sized by the largest layer.

* ``fprop(x, w)``, ``bprop(g, w, n)``, ``accgrad(x, g, k)`` -- the three
  operations (binary32, NCHW).
* ``r2c``, ``c2r``, ``cmul`` -- the stages, for tests and measurement.
* ``FrequencyBuffer`` -- the reused frequency-domain memory.
* ``FFTConv2dFn`` / ``FFTConv2d`` -- an autograd function and module that
  keep x and w only and recompute every transform in the backward.

Argument marshalling only; every element is computed by the HIP kernels.
"""

from __future__ import annotations

import torch
import torch.nn as nn

from . import _lib
from .functional import _require_device, _stream
from .dense import _current

SIZES = (8, 16, 32, 64)


def bins(n: int) -> int:
    return n * (n // 2 + 1)


class FrequencyBuffer:
    """Device memory for the spectra of one layer at a time; grows to the
    largest layer it serves and is never shrunk.  Kernels use it in stream
    order, so one buffer serves one stream at a time."""

    def __init__(self):
        self._t: torch.Tensor | None = None

    def get(self, nbytes: int, device) -> torch.Tensor:
        dev = torch.device(device)
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        t = self._t
        if t is None or t.numel() < nbytes or t.device != dev:
            self._t = t = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        return t

    @property
    def nbytes(self) -> int:
        return 0 if self._t is None else self._t.numel()


def _f32(t: torch.Tensor, name: str) -> torch.Tensor:
    _require_device(t, name)
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    return t.contiguous()


def _buffer(S, f, fo, n, device, buf):
    nbytes = _lib.library().fftconv_buffer_bytes(S, f, fo, n)
    if nbytes == 0:
        raise ValueError(f"unsupported sizes S={S} f={f} f'={fo} n={n} (n in {SIZES})")
    return (buf or FrequencyBuffer()).get(nbytes, device)


def _op(name, a, b, out, S, f, fo, n, k, buf):
    fb = _buffer(S, f, fo, n, a.device, buf)
    with _current(a.device):
        st = getattr(_lib.library(), name)(a.data_ptr(), b.data_ptr(), out.data_ptr(), S, f, fo, n,
                                           k, fb.data_ptr(), fb.numel(), _stream(a.device))
    _lib.check(st, name)
    return out


def fprop(x: torch.Tensor, w: torch.Tensor, buf: FrequencyBuffer | None = None) -> torch.Tensor:
    """y[s, f'] = sum_f x[s, f] (*) w[f', f] (valid cross-correlation)."""
    x, w = _f32(x, "x"), _f32(w, "w")
    S, f, n, n2 = x.shape
    fo, f2, k, k2 = w.shape
    if n != n2 or k != k2 or f != f2:
        raise ValueError(f"shapes x {tuple(x.shape)} and w {tuple(w.shape)} do not match")
    m = n - k + 1
    y = torch.empty((S, fo, m, m), dtype=torch.float32, device=x.device)
    return _op("fftconv_fprop", x, w, y, S, f, fo, n, k, buf)


def bprop(g: torch.Tensor, w: torch.Tensor, n: int, buf: FrequencyBuffer | None = None
          ) -> torch.Tensor:
    """gx[s, f] = sum_f' g[s, f'] (x) w[f', f] (full convolution), n x n."""
    g, w = _f32(g, "g"), _f32(w, "w")
    S, fo, m, m2 = g.shape
    fo2, f, k, k2 = w.shape
    if fo != fo2 or m != m2 or k != k2 or m != n - k + 1:
        raise ValueError(f"shapes g {tuple(g.shape)} and w {tuple(w.shape)} do not match n={n}")
    gx = torch.empty((S, f, n, n), dtype=torch.float32, device=g.device)
    return _op("fftconv_bprop", g, w, gx, S, f, fo, n, k, buf)


def accgrad(x: torch.Tensor, g: torch.Tensor, k: int, buf: FrequencyBuffer | None = None
            ) -> torch.Tensor:
    """gw[f', f] = sum_s x[s, f] (*) g[s, f'], k x k."""
    x, g = _f32(x, "x"), _f32(g, "g")
    S, f, n, n2 = x.shape
    S2, fo, m, m2 = g.shape
    if S != S2 or n != n2 or m != m2 or m != n - k + 1:
        raise ValueError(f"shapes x {tuple(x.shape)} and g {tuple(g.shape)} do not match k={k}")
    gw = torch.empty((fo, f, k, k), dtype=torch.float32, device=x.device)
    return _op("fftconv_accgrad", x, g, gw, S, f, fo, n, k, buf)


def r2c(maps: torch.Tensor, n: int) -> torch.Tensor:
    """Half spectra [bins, B] (complex64, bin-major) of B real m x m maps
    zero-padded to n x n."""
    maps = _f32(maps, "maps")
    B, m, m2 = maps.shape
    spec = torch.empty((bins(n), B), dtype=torch.complex64, device=maps.device)
    with _current(maps.device):
        st = _lib.library().fftconv_r2c(maps.data_ptr(), B, m, n, spec.data_ptr(),
                                        _stream(maps.device))
    _lib.check(st, "fftconv_r2c")
    return spec


def c2r(spec: torch.Tensor, n: int, m: int, scale: float) -> torch.Tensor:
    """The top-left m x m of the real inverse of half spectra [bins, B],
    times scale: [B, m, m]."""
    _require_device(spec, "spec")
    if spec.dtype != torch.complex64 or spec.dim() != 2 or spec.shape[0] != bins(n):
        raise ValueError(f"spec must be complex64 [{bins(n)}, B]")
    spec = spec.contiguous()
    B = spec.shape[1]
    y = torch.empty((B, m, m), dtype=torch.float32, device=spec.device)
    with _current(spec.device):
        st = _lib.library().fftconv_c2r(spec.data_ptr(), B, n, m, float(scale), y.data_ptr(),
                                        _stream(spec.device))
    _lib.check(st, "fftconv_c2r")
    return y


def cmul(op: int, a: torch.Tensor, b: torch.Tensor, S: int, f: int, fo: int) -> torch.Tensor:
    """The per-bin products (op 0 forward, 1 input gradient, 2 weight
    gradient) on bin-major spectra [bins, maps]."""
    for t, nm in ((a, "a"), (b, "b")):
        _require_device(t, nm)
        if t.dtype != torch.complex64 or t.dim() != 2:
            raise ValueError(f"{nm} must be complex64 [bins, maps]")
    P = a.shape[0]
    cols = {0: S * fo, 1: S * f, 2: fo * f}[op]
    c = torch.empty((P, cols), dtype=torch.complex64, device=a.device)
    with _current(a.device):
        st = _lib.library().fftconv_cmul(op, a.contiguous().data_ptr(), b.contiguous().data_ptr(),
                                         c.data_ptr(), S, f, fo, P, _stream(a.device))
    _lib.check(st, "fftconv_cmul")
    return c


class FFTConv2dFn(torch.autograd.Function):
    """y = conv(x, w) through FFTs; keeps x and w, recomputes every
    transform in the backward (nothing stays in the frequency domain)."""

    @staticmethod
    def forward(ctx, x, w, buf):
        ctx.buf = buf
        ctx.save_for_backward(x, w)
        return fprop(x, w, buf)

    @staticmethod
    def backward(ctx, g):
        x, w = ctx.saved_tensors
        g = g.contiguous()
        gx = bprop(g, w, x.shape[-1], ctx.buf) if ctx.needs_input_grad[0] else None
        gw = accgrad(x, g, w.shape[-1], ctx.buf) if ctx.needs_input_grad[1] else None
        return gx, gw, None


class FFTConv2d(nn.Module):
    """A convolution layer (no bias, stride 1, no padding) computed through
    FFTs, sharing a FrequencyBuffer with other layers."""

    def __init__(self, in_channels: int, out_channels: int, kernel_size: int,
                 buf: FrequencyBuffer | None = None):
        super().__init__()
        self.weight = nn.Parameter(torch.empty(out_channels, in_channels, kernel_size, kernel_size))
        nn.init.kaiming_normal_(self.weight)
        self.buf = buf or FrequencyBuffer()

    def forward(self, x):
        return FFTConv2dFn.apply(x, self.weight, self.buf)
