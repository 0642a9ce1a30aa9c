"""Tensor-level calls into libmeswish, named after the C ABI.

* ``swish_fwd(x, alpha)`` -> y = x * Sigmoid(alpha x)
  (blog post "Memory efficient Swish", "How is Swish implemented?").
* ``swish_bwd(x, dy, alpha)`` -> dy * s * (1 + t (1 - s)), t = alpha x,
  s = Sigmoid(t), from the saved input alone ("How is the memory efficient
  version Swish implemented?").
* ``swish_fwd_grouped`` / ``swish_bwd_grouped``: the same over a list of
  tensors in one launch per call (lists longer than 64 are split into calls
  of at most 64 tensors).

These functions only check and marshal arguments (device, dtype, shape,
contiguity, stream); they launch on the tensors' current HIP stream and
return without synchronising.  Tensors must live on a HIP device: there is
no CPU path.
"""

from __future__ import annotations

from typing import Sequence

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"libmeswish supports float32 and bfloat16, got {t.dtype}") from None


def _require_device(t: torch.Tensor, name: str) -> None:
    if t.device.type != "cuda":
        raise RuntimeError(f"{name} must be on a HIP (ROCm) device, got {t.device}; "
                           "libmeswish has no CPU path")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _same(a: torch.Tensor, b: torch.Tensor, an: str, bn: str) -> None:
    if a.device != b.device:
        raise ValueError(f"{an} and {bn} are on different devices")
    if a.dtype != b.dtype:
        raise TypeError(f"{an} and {bn} have different dtypes ({a.dtype}, {b.dtype})")
    if a.shape != b.shape:
        raise ValueError(f"{an} and {bn} have different shapes ({tuple(a.shape)}, {tuple(b.shape)})")


def _out(x: torch.Tensor, out: torch.Tensor | None, name: str) -> torch.Tensor:
    if out is None:
        return torch.empty_like(x, memory_format=torch.contiguous_format)
    _same(x, out, "x", name)
    if not out.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return out


def swish_fwd(x: torch.Tensor, alpha: float = 1.0, out: torch.Tensor | None = None) -> torch.Tensor:
    """y = x * sigmoid(alpha * x), computed by the gfx950 kernel."""
    _require_device(x, "x")
    code = _dtype_code(x)
    x = x.contiguous()
    y = _out(x, out, "out")
    with torch.cuda.device(x.device):
        st = _lib.library().swish_fwd(x.data_ptr(), y.data_ptr(), x.numel(), float(alpha), code,
                                      _stream(x.device))
    _lib.check(st, "swish_fwd")
    return y


def swish_bwd(x: torch.Tensor, dy: torch.Tensor, alpha: float = 1.0,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """dx = dy * s * (1 + t (1 - s)) with t = alpha x, s = sigmoid(t)."""
    _require_device(x, "x")
    _require_device(dy, "dy")
    _same(x, dy, "x", "dy")
    code = _dtype_code(x)
    x = x.contiguous()
    dy = dy.contiguous()
    dx = _out(x, out, "out")
    with torch.cuda.device(x.device):
        st = _lib.library().swish_bwd(x.data_ptr(), dy.data_ptr(), dx.data_ptr(), x.numel(),
                                      float(alpha), code, _stream(x.device))
    _lib.check(st, "swish_bwd")
    return dx


def _group_checks(xs: Sequence[torch.Tensor]) -> int:
    if len(xs) == 0:
        return _lib.F32
    for i, x in enumerate(xs):
        _require_device(x, f"xs[{i}]")
        if x.device != xs[0].device or x.dtype != xs[0].dtype:
            raise ValueError("all tensors of a group must share device and dtype")
    return _dtype_code(xs[0])


def swish_fwd_grouped(xs: Sequence[torch.Tensor], alpha: float = 1.0,
                      outs: Sequence[torch.Tensor] | None = None) -> list[torch.Tensor]:
    """Forward over several tensors, one kernel launch per (up to) 64 tensors."""
    code = _group_checks(xs)
    xs = [x.contiguous() for x in xs]
    ys = [_out(x, None if outs is None else outs[i], f"outs[{i}]") for i, x in enumerate(xs)]
    if not xs:
        return ys
    lib = _lib.library()
    with torch.cuda.device(xs[0].device):
        stream = _stream(xs[0].device)
        for lo in range(0, len(xs), _lib.MAX_GROUP):
            chunk = range(lo, min(lo + _lib.MAX_GROUP, len(xs)))
            desc = (_lib.FwdDesc * len(chunk))(
                *[_lib.FwdDesc(xs[j].data_ptr(), ys[j].data_ptr(), xs[j].numel()) for j in chunk])
            _lib.check(lib.swish_fwd_grouped(desc, len(chunk), float(alpha), code, stream),
                       "swish_fwd_grouped")
    return ys


def swish_bwd_grouped(xs: Sequence[torch.Tensor], dys: Sequence[torch.Tensor], alpha: float = 1.0,
                      outs: Sequence[torch.Tensor] | None = None) -> list[torch.Tensor]:
    """Backward over several tensors, one kernel launch per (up to) 64 tensors."""
    if len(xs) != len(dys):
        raise ValueError("xs and dys must have the same length")
    code = _group_checks(xs)
    for i, (x, dy) in enumerate(zip(xs, dys)):
        _require_device(dy, f"dys[{i}]")
        _same(x, dy, f"xs[{i}]", f"dys[{i}]")
    xs = [x.contiguous() for x in xs]
    dys = [d.contiguous() for d in dys]
    dxs = [_out(x, None if outs is None else outs[i], f"outs[{i}]") for i, x in enumerate(xs)]
    if not xs:
        return dxs
    lib = _lib.library()
    with torch.cuda.device(xs[0].device):
        stream = _stream(xs[0].device)
        for lo in range(0, len(xs), _lib.MAX_GROUP):
            chunk = range(lo, min(lo + _lib.MAX_GROUP, len(xs)))
            desc = (_lib.BwdDesc * len(chunk))(
                *[_lib.BwdDesc(xs[j].data_ptr(), dys[j].data_ptr(), dxs[j].data_ptr(),
                               xs[j].numel()) for j in chunk])
            _lib.check(lib.swish_bwd_grouped(desc, len(chunk), float(alpha), code, stream),
                       "swish_bwd_grouped")
    return dxs


def _act_code(kind: str) -> int:
    try:
        return _lib.ACTS[kind]
    except KeyError:
        raise ValueError(f"unknown activation {kind!r}; one of {sorted(_lib.ACTS)}") from None


def act_fwd(kind: str, x: torch.Tensor, param: float | None = None,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """y = f(x) for an activation of the family ("What activations cost, in
    memory and in arithmetic", Given): swish, relu, leaky_relu, sigmoid,
    tanh, gelu (erf), gelu_tanh.  ``param`` is Swish's alpha (default 1) or
    LeakyReLU's negative slope (default 0.01)."""
    code = _act_code(kind)
    p = _lib.DEFAULT_PARAM.get(kind, 0.0) if param is None else float(param)
    _require_device(x, "x")
    dt = _dtype_code(x)
    x = x.contiguous()
    y = _out(x, out, "out")
    with torch.cuda.device(x.device):
        st = _lib.library().meswish_act_fwd(code, x.data_ptr(), y.data_ptr(), x.numel(), p, dt,
                                            _stream(x.device))
    _lib.check(st, f"meswish_act_fwd({kind})")
    return y


def act_bwd(kind: str, x: torch.Tensor, dy: torch.Tensor, param: float | None = None,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """dx = dy f'(x), recomputed from the saved input x alone."""
    code = _act_code(kind)
    p = _lib.DEFAULT_PARAM.get(kind, 0.0) if param is None else float(param)
    _require_device(x, "x")
    _require_device(dy, "dy")
    _same(x, dy, "x", "dy")
    dt = _dtype_code(x)
    x = x.contiguous()
    dy = dy.contiguous()
    dx = _out(x, out, "out")
    with torch.cuda.device(x.device):
        st = _lib.library().meswish_act_bwd(code, x.data_ptr(), dy.data_ptr(), dx.data_ptr(),
                                            x.numel(), p, dt, _stream(x.device))
    _lib.check(st, f"meswish_act_bwd({kind})")
    return dx


def copy_bytes(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Plain 16-byte-vector device copy (bandwidth ceiling and counter calibration)."""
    _require_device(src, "src")
    _require_device(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    with torch.cuda.device(src.device):
        st = _lib.library().meswish_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream(src.device))
    _lib.check(st, "meswish_copy")
