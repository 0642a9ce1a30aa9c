"""Every pair of finite bfloat16 inputs (x, dy) of the backward of Swish
(alpha = 1) and of each activation of the family (LeakyReLU slope 0.01):
65,280 x 65,280 = 4,261,478,400 pairs each, through the C ABI, against the
binary64 oracle rounded to bfloat16 (rule: within one bfloat16 step, NaN
exactly where the oracle gives NaN).  Chunks of 4096 dy values against all
x; outputs bitwise equal to the oracle's are exact, the rest are counted."""

import time

import numpy as np
import pytest
import torch

import memory_efficient_activation_amd as mea
from memory_efficient_activation_amd import inputs
from oracle.compare import bf16_report

from gpu_util import ORACLE_THREADS, say

pytestmark = pytest.mark.gpu

DY_PER_CHUNK = 4096


FAMILY = ["relu", "leaky_relu", "sigmoid", "tanh", "gelu", "gelu_tanh"]
ORACLE_NAME = {"gelu": "gelu_erf"}
PARAM = {"leaky_relu": 0.01}


@pytest.mark.timeout(900)
def test_every_bf16_pair_backward(oracle):
    _pairs("swish", lambda x, dy: mea.swish_bwd(x, dy, 1.0),
           lambda xh, dyh: oracle.bwd(xh, dyh, 1.0, threads=ORACLE_THREADS, want_scale=False)[0])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kind", FAMILY)
def test_every_bf16_pair_backward_family(kind, oracle):
    p, oname = PARAM.get(kind, 0.0), ORACLE_NAME.get(kind, kind)
    _pairs(kind, lambda x, dy: mea.act_bwd(kind, x, dy, p),
           lambda xh, dyh: oracle.act_bwd(oname, xh, dyh, p, threads=ORACLE_THREADS,
                                          want_scale=False)[0])


def _pairs(label, gpu_bwd, oracle_bwd):
    dev = torch.device("cuda:0")
    xs = inputs.exhaustive_bf16_finite()               # uint16 bit patterns
    nx = xs.size
    assert nx == 65280
    x_dev = torch.from_numpy(xs.view(np.int16)).to(dev).view(torch.bfloat16)
    t0 = time.perf_counter()
    off_by_one = 0
    for c0 in range(0, nx, DY_PER_CHUNK):
        dys = xs[c0:c0 + DY_PER_CHUNK]
        k = dys.size
        xd = x_dev.repeat(k)
        dyd = torch.from_numpy(dys.view(np.int16)).to(dev).view(torch.bfloat16)
        dyd = dyd.repeat_interleave(nx)
        got = gpu_bwd(xd, dyd).view(torch.int16).cpu().numpy().view(np.uint16)
        del xd, dyd
        xh = np.tile(xs, k)
        dyh = np.repeat(dys, nx)
        want = oracle_bwd(xh, dyh)
        diff = np.nonzero(got != want)[0]
        r = bf16_report(got[diff], want[diff])
        off_by_one += r["n_off_by_one"]
        say(f"[bf16 pairs] {label} dy {c0}..{c0 + k - 1}: {diff.size} not bitwise equal, max "
            f"{r['max_ulp']} ulp ({time.perf_counter() - t0:.0f} s)")
        assert r["ok"], (c0, r, int(xh[diff[r["first_bad"]]]), int(dyh[diff[r["first_bad"]]]))
    say(f"[bf16 pairs] {label}: all {nx * nx} (x, dy) pairs, {off_by_one} one step off, "
        f"none more")
