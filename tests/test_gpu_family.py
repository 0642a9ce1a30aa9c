"""GPU parity of the activation family ("What activations cost, in memory
and in arithmetic", Given) through meswish_act_fwd / meswish_act_bwd.

Same rules as Swish (oracle/compare.py): binary32 within 1e-5 relative
(backward against the oracle's term-size scale), bfloat16 within 1 ulp,
NaN <-> NaN.  Inputs:

* the transformer-scale bfloat16 tensor [8, 2048, 4096] at full size (the
  benchmark's workload), x ~ N(0,1), dy ~ 0.01 N(0,1);
* a broad mixture (3 N(0,1) plus 2 % uniform in [-120, 120]) at a ragged
  length, both dtypes;
* every finite bfloat16 pattern, and every 4099th binary32 pattern;
* dense sweeps of each activation's rare branch;
* lengths 0..40 at misaligned offsets.
"""

import numpy as np
import pytest
import torch

import memory_efficient_activation_amd as mea
from memory_efficient_activation_amd import inputs
from oracle.compare import bf16_report, f32_report

from gpu_util import ORACLE_THREADS, say, to_dev, to_host

pytestmark = pytest.mark.gpu

FAMILY = ["relu", "leaky_relu", "sigmoid", "tanh", "gelu", "gelu_tanh"]
ORACLE_NAME = {"gelu": "gelu_erf"}
PARAM = {"leaky_relu": 0.01}


def _oname(kind):
    return ORACLE_NAME.get(kind, kind)


def _check(kind, xh, dyh, oracle, param=None, label=""):
    p = PARAM.get(kind, 0.0) if param is None else param
    x, dy = to_dev(xh), to_dev(dyh)
    y = mea.act_fwd(kind, x, p)
    dx = mea.act_bwd(kind, x, dy, p)
    torch.cuda.synchronize()
    oy = oracle.act_fwd(_oname(kind), xh, p, threads=ORACLE_THREADS)
    odx, m = oracle.act_bwd(_oname(kind), xh, dyh, p, threads=ORACLE_THREADS)
    if xh.dtype == np.uint16:
        rf, rb = bf16_report(to_host(y), oy), bf16_report(to_host(dx), odx)
    else:
        rf, rb = f32_report(to_host(y), oy), f32_report(to_host(dx), odx, m)
    if label:
        say(f"[family] {kind} {label}: fwd {rf} bwd {rb}")
    assert rf["ok"], (kind, label, rf)
    assert rb["ok"], (kind, label, rb)
    return rf, rb


@pytest.fixture(scope="module")
def workload3():
    return inputs.make(3)


@pytest.mark.parametrize("kind", FAMILY)
def test_family_full_size_bf16(kind, workload3, oracle):
    _check(kind, workload3.xs[0], workload3.dys[0], oracle, label="[8,2048,4096] bf16")


def _mixture(n, dtype, seed):
    rng = np.random.default_rng(seed)
    x = 3.0 * rng.standard_normal(n)
    m = rng.random(n) < 0.02
    x = np.where(m, rng.uniform(-120, 120, n), x)
    x[:6] = [0.0, -0.0, 1e-30, -1e-30, 0.125, -0.125]
    dy = rng.standard_normal(n)
    return inputs.encode(x, dtype), inputs.encode(dy, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", FAMILY)
def test_family_mixture(kind, dtype, oracle):
    xh, dyh = _mixture((1 << 20) + 13, dtype, 3)
    _check(kind, xh, dyh, oracle, label=f"mixture {dtype}")


@pytest.mark.parametrize("kind", FAMILY)
def test_family_exhaustive_bf16(kind, oracle):
    xb = inputs.exhaustive_bf16_finite()
    for dyv in (1.0, -0.01):
        dyb = inputs.encode(np.full(xb.size, dyv), "bf16")
        _check(kind, xb, dyb, oracle, label=f"all bf16, dy={dyv}")


@pytest.mark.parametrize("kind", FAMILY)
def test_family_fp32_patterns(kind, oracle):
    x = inputs.fp32_pattern_sample(4099)
    dy = np.random.default_rng(5).standard_normal(x.size).astype(np.float32)
    _check(kind, x, dy, oracle, label="fp32 patterns")


RARE_RANGES = {
    "sigmoid": [(-110.0, -80.0), (80.0, 110.0)],
    "tanh": [(38.0, 60.0), (-60.0, -38.0), (-0.2, 0.2)],
    "gelu": [(-16.0, -4.0), (4.0, 12.0)],
    "gelu_tanh": [(-14.0, -3.0), (3.0, 14.0)],
    "relu": [(-1.0, 1.0)],
    "leaky_relu": [(-1.0, 1.0)],
}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", FAMILY)
def test_family_rare_branches(kind, dtype, oracle):
    rng = np.random.default_rng(7)
    xs = [rng.uniform(lo, hi, 100000) for lo, hi in RARE_RANGES[kind]]
    x = np.concatenate(xs)
    dy = np.concatenate([rng.standard_normal(x.size - 6), [3e38, -3e38, 1e-30, -1e-40, 0.0, 1e20]])
    _check(kind, inputs.encode(x, dtype), inputs.encode(dy, dtype), oracle,
           label=f"rare-branch sweep {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_family_lengths_and_offsets(dtype, oracle):
    rng = np.random.default_rng(9)
    bx = inputs.encode(rng.standard_normal(256) * 4, dtype)
    bdy = inputs.encode(rng.standard_normal(256), dtype)
    xd, dyd = to_dev(bx), to_dev(bdy)
    out = torch.empty_like(xd)
    for kind in FAMILY:
        p = PARAM.get(kind, 0.0)
        for n in list(range(0, 41)) + [129]:
            for ox, oo in ((0, 0), (1, 1), (3, 1), (5, 0)):
                x, dy, y = xd[ox:ox + n], dyd[oo:oo + n], out[oo:oo + n]
                mea.act_fwd(kind, x, p, out=y)
                torch.cuda.synchronize()
                oy = oracle.act_fwd(_oname(kind), bx[ox:ox + n], p)
                r = (bf16_report if dtype == "bf16" else f32_report)(to_host(y), oy)
                assert r["ok"], (kind, n, ox, oo, r)
                mea.act_bwd(kind, x, dy, p, out=y)
                torch.cuda.synchronize()
                odx, m = oracle.act_bwd(_oname(kind), bx[ox:ox + n], bdy[oo:oo + n], p)
                got = to_host(y)
                r = bf16_report(got, odx) if dtype == "bf16" else f32_report(got, odx, m)
                assert r["ok"], (kind, n, ox, oo, r)


def test_swish_through_the_family_entry_points(oracle):
    w = inputs.make(4, n=1 << 20)
    x, dy = to_dev(w.xs[0]), to_dev(w.dys[0])
    a = mea.act_fwd("swish", x, w.alpha)
    b = mea.swish_fwd(x, w.alpha)
    c = mea.act_bwd("swish", x, dy, w.alpha)
    d = mea.swish_bwd(x, dy, w.alpha)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(c.view(torch.int32), d.view(torch.int32))


def test_leaky_relu_slope_and_swish_alpha_parameters(oracle):
    xh, dyh = _mixture(100003, "f32", 11)
    _check("leaky_relu", xh, dyh, oracle, param=0.2)
    _check("leaky_relu", xh, dyh, oracle, param=-1.5)


@pytest.mark.parametrize("kind", FAMILY)
def test_family_module_matches_torch_autograd(kind):
    """MemoryEfficientActivation against binary64 CPU autograd of torch's
    own activation."""
    import torch.nn.functional as F
    ref = {"relu": torch.relu, "leaky_relu": lambda t: F.leaky_relu(t, 0.01),
           "sigmoid": torch.sigmoid, "tanh": torch.tanh,
           "gelu": lambda t: F.gelu(t, approximate="none"),
           "gelu_tanh": lambda t: F.gelu(t, approximate="tanh")}[kind]
    rng = np.random.default_rng(13)
    # torch's own binary64 GELU cancels (1 + erf) below about -5: stay inside.
    xh = np.clip(rng.standard_normal(4099) * 1.5, -4.0, 4.0).astype(np.float32)
    dyh = rng.standard_normal(4099).astype(np.float32)
    x = torch.from_numpy(xh).cuda().requires_grad_(True)
    y = mea.MemoryEfficientActivation(kind, PARAM.get(kind))(x)
    y.backward(torch.from_numpy(dyh).cuda())
    xr = torch.from_numpy(xh.astype(np.float64)).requires_grad_(True)
    yr = ref(xr)
    yr.backward(torch.from_numpy(dyh.astype(np.float64)))
    torch.cuda.synchronize()
    assert np.allclose(to_host(y).astype(np.float64), yr.detach().numpy(), rtol=2e-6, atol=1e-30)
    gd = to_host(x.grad).astype(np.float64)
    gr = xr.grad.numpy()
    assert np.allclose(gd, gr, rtol=1e-5, atol=2e-6 * np.abs(dyh).max())
