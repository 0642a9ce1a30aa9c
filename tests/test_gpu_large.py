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

The DenseNet stage gets the same treatment: a source and a shared map past
2^31 elements, with sampled channels checked against its binary64 oracle.
"""

import numpy as np
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


N32 = (1 << 32) + 4097  # bf16 elements: 8 GiB + 8 KiB per tensor


def test_bf16_element_path_past_2_32_elements(oracle):
    """x 2 bytes past alignment, y and dy aligned: the element-wise kernels on
    n = 2^32 + 4097 elements, where one thread per 256-element tile would need
    a grid of more than 2^32 threads.  The host caps the grid (the kernels
    loop over the rest); sampled outputs at the start, around 2^31 and 2^32,
    at the end and 200,000 uniform indices match the oracle."""
    say(f"[large] bf16 element path n={N32}")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(31)
    xb = torch.empty(N32 + 1, dtype=torch.bfloat16, device=dev)
    xb.normal_(0.0, 4.0, generator=g)
    x = xb[1:]
    dy = torch.empty(N32, dtype=torch.bfloat16, device=dev)
    dy.normal_(0.0, 1.0, generator=g)
    x[(1 << 32) - 1] = -30.0
    x[1 << 32] = 7.5
    y = torch.empty(N32, dtype=torch.bfloat16, device=dev)
    mea.swish_fwd(x, 1.0, out=y)
    dx = torch.empty(N32, dtype=torch.bfloat16, device=dev)
    mea.swish_bwd(x, dy, 1.0, out=dx)
    torch.cuda.synchronize()
    idx = torch.cat([torch.arange(0, 2048), torch.arange((1 << 31) - 2048, (1 << 31) + 2048),
                     torch.arange((1 << 32) - 4096, (1 << 32) + 4096), torch.arange(N32 - 4096, N32),
                     torch.randint(0, N32, (200000,), generator=torch.Generator().manual_seed(7))])
    idx = idx.to(dev)
    xs, dys = to_host(x[idx]), to_host(dy[idx])
    ry = bf16_report(to_host(y[idx]), oracle.fwd(xs, 1.0, threads=ORACLE_THREADS))
    odx, _ = oracle.bwd(xs, dys, 1.0, threads=ORACLE_THREADS, want_scale=False)
    rdx = bf16_report(to_host(dx[idx]), odx)
    say(f"[large] bf16 element path past 2^32: fwd {ry} bwd {rdx}")
    assert ry["ok"], ry
    assert rdx["ok"], rdx
    del xb, x, dy, y, dx


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


def test_dense_stage_past_2_31_elements(oracle):
    """The DenseNet stage (include/dense_bn.h) on two binary32 sources of 1040
    and 24 channels, n = 2 rows of hw = 2^20 each: the first source holds
    2,181,038,080 elements, the shared map z 2,231,369,728 (both past 2^31,
    8.7 and 8.9 GB).  Per channel there are 2^21 elements, inside the stage's
    limit.  Seven channels at the ends and middle of both sources are checked
    against the binary64 oracle: statistics, z, dx, dgamma, dbeta (channels
    are independent, so the oracle takes them as one small layer)."""
    from memory_efficient_activation_amd import dense
    from oracle import dense_oracle as do

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(31)
    n, hw, chans = 2, 1 << 20, (1040, 24)
    say(f"[large] dense stage: sources {chans} x n={n} x hw={hw}, binary32")
    xs = []
    for c in chans:
        off = torch.randn(c, device=dev, generator=g)
        sc = torch.rand(c, device=dev, generator=g) * 1.5 + 0.5
        x = torch.empty((n, c, hw), device=dev)
        x.normal_(generator=g)
        x.mul_(sc[None, :, None]).add_(off[None, :, None])
        xs.append(x)
    total = sum(chans)
    gamma = 1.0 + 0.25 * torch.randn(total, device=dev, generator=g)
    beta = 0.5 * torch.randn(total, device=dev, generator=g)
    dz = torch.empty((n, total, hw), device=dev)
    dz.normal_(generator=g)
    eps = dense.EPS
    stats = [dense.bn_stats(x) for x in xs]
    z = dense.bn_relu_fwd(xs, stats, gamma, beta, eps)
    dxs, dg, db = dense.bn_relu_bwd(xs, stats, gamma, beta, dz, eps)
    torch.cuda.synchronize()

    picks = [(0, 0), (0, 1), (0, 517), (0, 1038), (0, 1039), (1, 0), (1, 23)]
    zc = [sum(chans[:j]) + c for j, c in picks]
    src = np.stack([to_host(xs[j][:, c, :]).astype(np.float64) for j, c in picks], axis=1)
    g64 = to_host(gamma)[zc].astype(np.float64)
    b64 = to_host(beta)[zc].astype(np.float64)
    dz64 = np.stack([to_host(dz[:, c, :]).astype(np.float64) for c in zc], axis=1)
    zo, f = do.forward([src], g64, b64, eps)
    duo, dgo, dbo, aux = do.backward([src], dz64, g64, b64, eps)

    mean = np.array([to_host(stats[j][c, 0]) for j, c in picks])
    var = np.array([to_host(stats[j][c, 1]) for j, c in picks])
    mean_err = float((np.abs(mean - f["mean"]) / (np.abs(f["mean"]) + np.sqrt(f["var"]))).max())
    var_err = float((np.abs(var - f["var"]) / f["var"]).max())
    say(f"[large] dense stats: mean {mean_err:.2e}, var {var_err:.2e}")
    assert mean_err <= 1e-12 and var_err <= 1e-10

    zg = np.stack([to_host(z[:, c, :]) for c in zc], axis=1)
    rz = f32_report(zg, oracle.round_array(zo, "f32"), f["scale"], 1e-5)
    dxg = np.stack([to_host(dxs[j][:, c, :]) for j, c in picks], axis=1)
    rdx = f32_report(dxg, oracle.round_array(duo[0], "f32"), aux["du_scale"][0], 1e-5)
    rdg = f32_report(to_host(dg)[zc], dgo.astype(np.float32), aux["dgamma_scale"], 1e-5)
    rdb = f32_report(to_host(db)[zc], dbo.astype(np.float32), aux["dbeta_scale"], 1e-5)
    say(f"[large] dense z {rz['max_rel']:.2e}, dx {rdx['max_rel']:.2e}, "
        f"dgamma {rdg['max_rel']:.2e}, dbeta {rdb['max_rel']:.2e}")
    for r in (rz, rdx, rdg, rdb):
        assert r["ok"], r


def test_fft_transforms_near_the_size_limit():
    """FFT convolution's transforms (include/fft_conv.h) at the size limit:
    3,900,000 maps of 32 x 32 (15.6 GB) give half spectra of 2,121,600,000
    complex values (17 GB, bin-major), just under the limit of 2^31 per
    spectrum array, so offsets run past byte 2^34.  Sampled maps are checked
    against the oracle's transform (numpy FFT of the map); every map must come
    back from the inverse (the round trip, a property at any size) to within
    1e-5 of its norm."""
    from memory_efficient_activation_amd import fft
    from oracle import fft_oracle as fo_

    dev = torch.device("cuda:0")
    B, n = 3_900_000, 32
    say(f"[large] fft: r2c + c2r of {B} maps of {n} x {n}, {fft.bins(n) * B} bins")
    g = torch.Generator(device=dev)
    g.manual_seed(37)
    x = torch.empty((B, n, n), device=dev)
    x.normal_(generator=g)
    spec = fft.r2c(x, n)
    torch.cuda.synchronize()
    idx = torch.cat([torch.tensor([0, 1, 2, B // 2, B - 3, B - 2, B - 1]),
                     torch.randint(0, B, (40,), generator=torch.Generator().manual_seed(3))])
    xs = to_host(x[idx.to(dev)]).astype(np.float64)
    got = to_host(spec[:, idx.to(dev)]).astype(np.complex128)           # [P, k]
    want = fo_.rfft2_half(xs, n).reshape(len(idx), -1).T
    err = float((np.abs(got - want).max(0) / fo_.spectrum_scale(xs, n)).max())
    say(f"[large] fft r2c, sampled maps: max err / (n ||x||) = {err:.2e}")
    assert err <= 1e-5

    y = fft.c2r(spec, n, n, 1.0 / (n * n))
    del spec
    worst = 0.0
    for c0 in range(0, B, 500_000):
        xc, yc = x[c0:c0 + 500_000], y[c0:c0 + 500_000]
        d = (yc - xc).abs().amax(dim=(1, 2)) / xc.norm(dim=(1, 2))
        worst = max(worst, float(d.max()))
    say(f"[large] fft round trip, all maps: max |y - x| / ||x|| = {worst:.2e}")
    assert worst <= 1e-5
