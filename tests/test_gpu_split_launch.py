"""The split of one tensor into several launches, on the GPU.

The library splits a tensor whose vector body has more than 2^30 tiles into
several launches (the kernels index tiles with 32-bit integers).  Tensors
that large take 64 GiB and more, so this file runs the same host code in a
test build with 3 tiles per launch (``libmeswish_split3.so``, made by
``__graft_entry__.build()``), where a tensor of a few thousand elements
already takes several launches.  Each output, for starts 0 to 15 bytes past
a 16-byte boundary (a scalar head in the first launch) and ragged lengths (a
scalar tail in the last), must equal the single-launch library bit for bit
and the oracle to the parity bar (1e-5 of the scale in binary32, one unit in
the last place in bfloat16).
"""

import ctypes

import pytest
import torch

import memory_efficient_activation_amd as mea
from memory_efficient_activation_amd import _lib
from memory_efficient_activation_amd import build as lib_build
from oracle.compare import bf16_report, f32_report

from gpu_util import ORACLE_THREADS, say, to_host

pytestmark = pytest.mark.gpu

SIZES = [1, 7, 100, 2049, 5000, 9 * 512 + 7, 40000, 1_000_003]


@pytest.fixture(scope="module")
def lib3():
    import os
    if not os.path.exists(lib_build.SPLIT_TEST_LIBRARY):
        pytest.fail("the split test build is missing (run __graft_entry__.build())")
    return _lib.library(lib_build.SPLIT_TEST_LIBRARY, lib_build.SPLIT_TEST_NAMES)


def _views(n, dtype, shift, gen):
    """x, dy and an output buffer (NaN-filled), each starting ``shift`` elements past a
    256-byte aligned allocation (congruent pointers: the vector path)."""
    def buf(scale):
        b = torch.randn(n + shift, generator=gen, device="cuda:0", dtype=torch.float32) * scale
        return b.to(dtype)[shift:]
    x, dy, out = buf(4.0), buf(1.0), buf(0.0)
    out.fill_(float("nan"))
    return x, dy, out


ORACLE_NAME = {"gelu": "gelu_erf"}


def _check(got, want, x, dy, kind, p, oracle, bwd):
    """Bitwise against the single-launch library, then against the oracle."""
    kind = ORACLE_NAME.get(kind, kind)
    assert torch.equal(got.view(torch.int16 if got.dtype == torch.bfloat16 else torch.int32),
                       want.view(torch.int16 if want.dtype == torch.bfloat16 else torch.int32))
    hx = to_host(x)
    if bwd:
        o, m = oracle.act_bwd(kind, hx, to_host(dy), p, threads=ORACLE_THREADS,
                              want_scale=got.dtype == torch.float32)
    else:
        o, m = oracle.act_fwd(kind, hx, p, threads=ORACLE_THREADS), None
    r = bf16_report(to_host(got), o) if got.dtype == torch.bfloat16 else \
        f32_report(to_host(got), o, m)
    assert r["ok"], r


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("kind,param", [("swish", 1.0), ("swish", 1.5), ("gelu", 0.0)])
def test_split_launches_equal_single_launch(lib3, dtype, kind, param, oracle):
    code = _lib.F32 if dtype == torch.float32 else _lib.BF16
    esize = 4 if dtype == torch.float32 else 2
    act = _lib.ACTS[kind]
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(11)
    stream = torch.cuda.current_stream().cuda_stream
    for n in SIZES:
        for shift in (0, 1, 16 // esize - 1):
            x, dy, out3 = _views(n, dtype, shift, gen)
            p = _lib.Plan()
            assert lib3.meswish_plan(x.data_ptr(), dy.data_ptr(), out3.data_ptr(), n, param, code,
                                     1, ctypes.byref(p)) == _lib.OK
            say(f"[split] {kind} p={param} {dtype} n={n} shift={shift}: "
                f"{p.tiles} tiles in {p.launches} launches")
            assert p.path == _lib.PATH_VECTOR
            assert p.launches == max(1, -(-p.tiles // lib_build.SPLIT_TEST_TILES))
            if kind == "swish":
                _lib.check(lib3.swish_fwd(x.data_ptr(), out3.data_ptr(), n, param, code, stream),
                           "swish_fwd (split build)")
                want = mea.swish_fwd(x, param)
            else:
                _lib.check(lib3.meswish_act_fwd(act, x.data_ptr(), out3.data_ptr(), n, param, code,
                                                stream), "meswish_act_fwd (split build)")
                want = mea.act_fwd(kind, x, param)
            torch.cuda.synchronize()
            _check(out3, want, x, dy, kind, param, oracle, False)
            out3.fill_(float("nan"))
            if kind == "swish":
                _lib.check(lib3.swish_bwd(x.data_ptr(), dy.data_ptr(), out3.data_ptr(), n, param,
                                          code, stream), "swish_bwd (split build)")
                want = mea.swish_bwd(x, dy, param)
            else:
                _lib.check(lib3.meswish_act_bwd(act, x.data_ptr(), dy.data_ptr(), out3.data_ptr(),
                                                n, param, code, stream),
                           "meswish_act_bwd (split build)")
                want = mea.act_bwd(kind, x, dy, param)
            torch.cuda.synchronize()
            _check(out3, want, x, dy, kind, param, oracle, True)


def test_split_leaves_neighbours_alone(lib3):
    """Each launch writes only its own part: guard elements on both sides of
    the output keep their values."""
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(3)
    stream = torch.cuda.current_stream().cuda_stream
    for dtype, code in ((torch.float32, _lib.F32), (torch.bfloat16, _lib.BF16)):
        for n, lead in ((5000, 3), (40000, 0), (2049, 1)):
            x = (torch.randn(n, generator=gen, device="cuda:0") * 4).to(dtype)
            guard = torch.full((n + lead + 64,), 7.0, device="cuda:0", dtype=dtype)
            x2 = torch.empty_like(guard)
            x2[lead:lead + n] = x
            xs = x2[lead:lead + n]
            out = guard[lead:lead + n]
            _lib.check(lib3.swish_fwd(xs.data_ptr(), out.data_ptr(), n, 1.0, code, stream),
                       "swish_fwd (split build)")
            torch.cuda.synchronize()
            assert bool((guard[:lead] == 7.0).all()) and bool((guard[lead + n:] == 7.0).all())
            assert torch.equal(out.float(), mea.swish_fwd(xs, 1.0).float())
