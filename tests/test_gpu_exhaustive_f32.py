"""Every binary32 input x of Swish and of the activation family, through the
C ABI, against the binary64 oracle rounded to binary32: all 2^32 bit
patterns (normal, subnormal, zero, infinite and NaN).  Swish: the forward at
alpha = 1 and 1.5 and the backward at alpha = 1 with dy = 1 and dy = -0.3;
the family: forward and backward with dy = 1 (LeakyReLU slope 0.01).  The rules are the binary32 ones:
forward within 1e-5 of |reference| (floored at 2^-126), backward within 1e-5
of the oracle's term scale m, NaN exactly where the oracle gives NaN.
Chunks of 2^28 patterns; outputs bitwise equal to the oracle's are exact, and
the rest go through the rule."""

import time

import numpy as np
import pytest
import torch

import memory_efficient_activation_amd as mea
from oracle.compare import f32_report

from gpu_util import ORACLE_THREADS, say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28


def _sweep(label, gpu_fn, oracle_fn):
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    total_diff, worst = 0, 0.0
    for c in range((1 << 32) // CHUNK):
        lo = -(1 << 31) + c * CHUNK
        x = torch.arange(lo, lo + CHUNK, dtype=torch.int32, device=dev).view(torch.float32)
        got = gpu_fn(x).view(torch.int32).cpu().numpy()
        del x
        xh = np.arange(lo, lo + CHUNK, dtype=np.int32).view(np.float32)
        want, scale = oracle_fn(xh)
        want = want.view(np.int32)
        diff = np.nonzero(got != want)[0]
        r = f32_report(got[diff].view(np.float32), want[diff].view(np.float32),
                       None if scale is None else scale[diff])
        total_diff += diff.size
        worst = max(worst, r["max_rel"])
        say(f"[exhaustive f32] {label} chunk {c + 1}/16: {diff.size} not bitwise equal, "
            f"max rel {r['max_rel']:.2e} ({time.perf_counter() - t0:.0f} s)")
        assert r["ok"], (label, c, r, int(xh[diff[r["first_bad"]]].view(np.uint32)))
    say(f"[exhaustive f32] {label}: all 2^32 x, {total_diff} differ in the last bits, "
        f"worst relative error {worst:.2e}, none outside the rule")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("alpha", [1.0, 1.5])
def test_every_binary32_x_forward(alpha, oracle):
    _sweep(f"forward alpha={alpha}", lambda x: mea.swish_fwd(x, alpha),
           lambda xh: (oracle.fwd(xh, alpha, threads=ORACLE_THREADS), None))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dy", [1.0, -0.3])
def test_every_binary32_x_backward(dy, oracle):
    def gpu(x):
        return mea.swish_bwd(x, torch.full_like(x, dy), 1.0)

    def ref(xh):
        return oracle.bwd(xh, np.full_like(xh, np.float32(dy)), 1.0, threads=ORACLE_THREADS)

    _sweep(f"backward dy={dy}", gpu, ref)


FAMILY = ["relu", "leaky_relu", "sigmoid", "tanh", "gelu", "gelu_tanh"]
ORACLE_NAME = {"gelu": "gelu_erf"}
PARAM = {"leaky_relu": 0.01}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kind", FAMILY)
def test_every_binary32_x_family(kind, oracle):
    """The activation family, forward and backward (dy = 1), every binary32 x."""
    p, oname = PARAM.get(kind, 0.0), ORACLE_NAME.get(kind, kind)
    _sweep(f"{kind} forward", lambda x: mea.act_fwd(kind, x, p),
           lambda xh: (oracle.act_fwd(oname, xh, p, threads=ORACLE_THREADS), None))

    def gpu(x):
        return mea.act_bwd(kind, x, torch.ones_like(x), p)

    def ref(xh):
        return oracle.act_bwd(oname, xh, np.ones_like(xh), p, threads=ORACLE_THREADS)

    _sweep(f"{kind} backward dy=1", gpu, ref)
