"""GPU parity on the five synthetic workloads, through the C ABI.

Every output element of the HIP path is compared with the CPU oracle on the
same seeded inputs:

* binary32: |g - o| <= 1e-5 * max(|o|, 2^-126) forward and
  |g - o| <= 1e-5 * max(m, 2^-126) backward (m: the oracle's error scale);
* bfloat16: at most 1 unit in the last place (ordered bit patterns).

Workloads run at full size, in the launch configuration the benchmark times
(the same library entry points), and also at reduced sizes that span several
tiles and a ragged tail.
"""

import numpy as np
import pytest
import torch

import memory_efficient_activation_amd as mea
from memory_efficient_activation_amd import inputs
from oracle.compare import bf16_report, f32_report

from gpu_util import ORACLE_THREADS, say, to_dev, to_host

pytestmark = pytest.mark.gpu

W0 = 1.2784645427610738  # |x| at the zero of Swish' for alpha = 1 (1 + W(1/e))


def _report(w, got, want, scale=None):
    if w.dtype == "bf16":
        return bf16_report(got, want)
    return f32_report(got, want, scale)


def _run_single(w, oracle, idx=0):
    x, dy = to_dev(w.xs[idx]), to_dev(w.dys[idx])
    y = mea.swish_fwd(x, w.alpha)
    dx = mea.swish_bwd(x, dy, w.alpha)
    torch.cuda.synchronize()
    gy, gdx = to_host(y), to_host(dx)
    oy = oracle.fwd(w.xs[idx], w.alpha, threads=ORACLE_THREADS)
    odx, m = oracle.bwd(w.xs[idx], w.dys[idx], w.alpha, threads=ORACLE_THREADS,
                        want_scale=w.dtype == "f32")
    rf = _report(w, gy, oy)
    rb = _report(w, gdx, odx, m)
    return rf, rb, (gdx, odx)


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_workload_full_size(index, oracle):
    w = inputs.make(index)
    say(f"[parity] workload {index}: {w.name}, n={w.numel}")
    rf, rb, (gdx, odx) = _run_single(w, oracle)
    say(f"[parity] workload {index} fwd {rf}")
    say(f"[parity] workload {index} bwd {rb}")
    if w.dtype == "f32":
        # Plain relative error of the backward away from the zero of Swish'.
        x = inputs.decode(w.xs[0]).astype(np.float64)
        t = w.alpha * x
        away = np.abs(np.abs(t) - W0) >= 0.05
        near = ~away
        o = odx.astype(np.float64)
        g = gdx.astype(np.float64)
        rel = np.abs(g - o)[away] / np.maximum(np.abs(o[away]), 2.0 ** -126)
        say(f"[parity] workload {index} bwd plain max rel outside |t-t0|<0.05: "
            f"{rel.max():.3e}; elements inside the band: {int(near.sum())}")
    assert rf["ok"], rf
    assert rb["ok"], rb


@pytest.mark.parametrize("index", [1, 2, 3, 4])
@pytest.mark.parametrize("n", [1, 3, 8, 9, 1000, 4096, 65537, 1 << 20, (1 << 20) + 13])
def test_workload_recipes_ragged_sizes(index, n, oracle):
    w = inputs.make(index, n=n)
    rf, rb, _ = _run_single(w, oracle)
    assert rf["ok"], (n, rf)
    assert rb["ok"], (n, rb)


def test_workload5_grouped_full_size(oracle):
    w = inputs.make(5)
    say(f"[parity] workload 5: {w.name}, n={w.numel}")
    xs = [to_dev(a) for a in w.xs]
    dys = [to_dev(a) for a in w.dys]
    ys = mea.swish_fwd_grouped(xs, w.alpha)
    dxs = mea.swish_bwd_grouped(xs, dys, w.alpha)
    # The same tensors one launch each: grouped must equal single bit for bit.
    ys1 = [mea.swish_fwd(x, w.alpha) for x in xs]
    dxs1 = [mea.swish_bwd(x, d, w.alpha) for x, d in zip(xs, dys)]
    torch.cuda.synchronize()
    worst_f, worst_b = 0, 0
    for i in range(len(xs)):
        oy = oracle.fwd(w.xs[i], w.alpha, threads=ORACLE_THREADS)
        odx, _ = oracle.bwd(w.xs[i], w.dys[i], w.alpha, threads=ORACLE_THREADS, want_scale=False)
        rf = bf16_report(to_host(ys[i]), oy)
        rb = bf16_report(to_host(dxs[i]), odx)
        say(f"[parity] workload 5 tensor {i} {w.shapes[i]}: fwd max_ulp={rf['max_ulp']} "
            f"bwd max_ulp={rb['max_ulp']}")
        assert rf["ok"], (i, rf)
        assert rb["ok"], (i, rb)
        worst_f, worst_b = max(worst_f, rf["max_ulp"]), max(worst_b, rb["max_ulp"])
        assert torch.equal(ys[i].view(torch.int16), ys1[i].view(torch.int16))
        assert torch.equal(dxs[i].view(torch.int16), dxs1[i].view(torch.int16))
    say(f"[parity] workload 5 worst fwd {worst_f} ulp, bwd {worst_b} ulp")
