"""Tensors past 2^31 elements and 4 GiB, through the C ABI, against the CPU
oracle on sampled elements.

The kernels index with 64-bit integers throughout; these cases make that
visible.  n = 2^31 + 12345 elements (4 GiB + 24 KiB in bfloat16, 8 GiB + 48 KiB
in binary32), so element 2^31 and byte 2^32 (and, for binary32, byte 2^33)
fall inside the tensor.  The paths covered: 16-byte vectors from an aligned
start, vectors after a scalar head (all pointers 6 bytes past alignment), the
element-wise path (input and output not congruent modulo 16), and the
grouped launch, which must equal single launches bit for bit.

Inputs come from torch's seeded device generator (x ~ 4 N(0,1), dy ~ N(0,1)),
with a few planted values next to 2^31 and in the ragged tail.  The samples
are the first elements, the neighbourhoods of 2^30 and 2^31, the last
elements and 200,000 uniform indices; the oracle computes each of them from
the sampled input.
"""

import pytest
import torch

import memory_efficient_activation_amd as mea
from oracle.compare import bf16_report, f32_report

from gpu_util import ORACLE_THREADS, say, to_host

pytestmark = pytest.mark.gpu

N = (1 << 31) + 12345
PLANTED = {(1 << 31) - 1: -100.0, 1 << 31: -0.0, (1 << 31) + 1: 30.0, N - 1: -30.0,
           N - 2: 1e-30, 1 << 30: -60.0, 5: 7.5}


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    torch.cuda.empty_cache()


def _inputs(dtype, offset, seed):
    """x, dy of N elements starting `offset` elements into their buffers."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    xb = torch.empty(N + 8, dtype=dtype, device=dev)
    db = torch.empty(N + 8, dtype=dtype, device=dev)
    xb.normal_(0.0, 4.0, generator=g)
    db.normal_(0.0, 1.0, generator=g)
    x, dy = xb[offset:offset + N], db[offset:offset + N]
    for i, v in PLANTED.items():
        x[i] = v
    return x, dy


def _sample_index(dev):
    parts = [torch.arange(0, 2048), torch.arange((1 << 30) - 2048, (1 << 30) + 2048),
             torch.arange((1 << 31) - 4096, (1 << 31) + 4096), torch.arange(N - 8192, N),
             torch.randint(0, N, (200000,), generator=torch.Generator().manual_seed(5))]
    return torch.cat(parts).to(dev)


def _check(x, dy, y, dx, alpha, oracle, what):
    idx = _sample_index(x.device)
    xs, ys = to_host(x[idx]), to_host(y[idx])
    oy = oracle.fwd(xs, alpha, threads=ORACLE_THREADS)
    if x.dtype == torch.bfloat16:
        ry = bf16_report(ys, oy)
    else:
        ry = f32_report(ys, oy)
    say(f"[large] {what} fwd: {ry}")
    assert ry["ok"], ry
    if dx is None:
        return
    dys, dxs = to_host(dy[idx]), to_host(dx[idx])
    odx, m = oracle.bwd(xs, dys, alpha, threads=ORACLE_THREADS)
    rdx = bf16_report(dxs, odx) if x.dtype == torch.bfloat16 else f32_report(dxs, odx, m)
    say(f"[large] {what} bwd: {rdx}")
    assert rdx["ok"], rdx


@pytest.mark.parametrize("offset", [0, 3])
def test_bf16_past_2_31_elements(offset, oracle):
    say(f"[large] bf16 n={N} offset={offset}")
    x, dy = _inputs(torch.bfloat16, offset, seed=11 + offset)
    yb = torch.empty(N + 8, dtype=torch.bfloat16, device=x.device)
    db = torch.empty(N + 8, dtype=torch.bfloat16, device=x.device)
    y, dx = yb[offset:offset + N], db[offset:offset + N]
    mea.swish_fwd(x, 1.0, out=y)
    mea.swish_bwd(x, dy, 1.0, out=dx)
    torch.cuda.synchronize()
    _check(x, dy, y, dx, 1.0, oracle, f"bf16 offset {offset}")


def test_bf16_element_path_past_2_31(oracle):
    """x 6 bytes past alignment, y aligned: the element-wise kernel."""
    say(f"[large] bf16 element path n={N}")
    x, dy = _inputs(torch.bfloat16, 3, seed=17)
    y = torch.empty(N, dtype=torch.bfloat16, device=x.device)
    mea.swish_fwd(x, 1.0, out=y)
    torch.cuda.synchronize()
    _check(x, dy, y, None, 1.0, oracle, "bf16 element path")


def test_grouped_equals_single_past_2_31():
    say(f"[large] grouped, one tensor of n={N} and one of 1000")
    x, dy = _inputs(torch.bfloat16, 0, seed=23)
    small = torch.linspace(-9, 9, 1000, device=x.device).to(torch.bfloat16)
    dsmall = torch.linspace(1, -1, 1000, device=x.device).to(torch.bfloat16)
    y1 = mea.swish_fwd(x, 0.8)
    ys = mea.swish_fwd_grouped([x, small], 0.8)
    assert torch.equal(ys[0].view(torch.int16), y1.view(torch.int16))
    del ys, y1
    d1 = mea.swish_bwd(x, dy, 0.8)
    ds = mea.swish_bwd_grouped([x, small], [dy, dsmall], 0.8)
    assert torch.equal(ds[0].view(torch.int16), d1.view(torch.int16))
    assert torch.equal(ds[1].view(torch.int16), mea.swish_bwd(small, dsmall, 0.8).view(torch.int16))
    torch.cuda.synchronize()


def test_f32_past_8_gib(oracle):
    say(f"[large] f32 n={N} ({4 * N} bytes per tensor)")
    x, dy = _inputs(torch.float32, 0, seed=29)
    y = mea.swish_fwd(x, 1.5)
    dx = mea.swish_bwd(x, dy, 1.5)
    torch.cuda.synchronize()
    _check(x, dy, y, dx, 1.5, oracle, "f32")
