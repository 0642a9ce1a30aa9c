"""Every path of libmeswish captured into a HIP graph.

The kernels take no memsets, allocations or host synchronisations, so a
caller may capture them.  Each case below captures one call sequence on a
side stream, replays it several times with eager work and synchronisations
between the replays, and requires every replay to give the eager result bit
for bit (inputs are static tensors; outputs are the graph's own)."""

import numpy as np
import pytest
import torch

import memory_efficient_activation_amd as mea
from memory_efficient_activation_amd import dense, dense_inputs as di, fft, fft_inputs, inputs

from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu
REPLAYS = 3


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _capture_and_check(fn, label):
    """fn() -> list of output tensors.  Eager result, then capture, replays."""
    eager = [o.clone() for o in fn()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = fn()
    for r in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else 0)  # stale values must not survive
        graph.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(_bits(a), _bits(b)), (label, r, k)
        torch.randn(1 << 18, device="cuda").sum().item()  # eager work between replays
    say(f"[graphs] {label}: {REPLAYS} replays equal to the eager result")
    del graph


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_swish_and_family(dtype):
    rng = np.random.default_rng(1)
    x = to_dev(inputs.encode(rng.standard_normal(100003) * 3, dtype))
    dy = to_dev(inputs.encode(rng.standard_normal(100003), dtype))

    def fn():
        outs = [mea.swish_fwd(x, 1.25), mea.swish_bwd(x, dy, 1.25)]
        for kind in ("relu", "leaky_relu", "sigmoid", "tanh", "gelu", "gelu_tanh"):
            outs += [mea.act_fwd(kind, x), mea.act_bwd(kind, x, dy)]
        return outs

    _capture_and_check(fn, f"swish and family, {dtype}")


def test_grouped_swish():
    rng = np.random.default_rng(2)
    xs = [to_dev(inputs.encode(rng.standard_normal(n), "bf16")) for n in (4099, 17, 65536, 3)]
    dys = [to_dev(inputs.encode(rng.standard_normal(x.numel()), "bf16")) for x in xs]

    def fn():
        return list(mea.swish_fwd_grouped(xs, 1.0)) + list(mea.swish_bwd_grouped(xs, dys, 1.0))

    _capture_and_check(fn, "grouped swish, bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_layer_stage(dtype):
    w = di.densenet_bc100_layer(1, 7, dtype, n=16)
    xs = [to_dev(s) for s in w.sources]
    gamma, beta, dz = to_dev(w.gamma), to_dev(w.beta), to_dev(w.dz)

    def fn():
        stats = [dense.bn_stats(x) for x in xs]
        z = dense.bn_relu_fwd(xs, stats, gamma, beta, w.eps)
        dxs, dg, db = dense.bn_relu_bwd(xs, stats, gamma, beta, dz, w.eps)
        return stats + [z] + list(dxs) + [dg, db]

    _capture_and_check(fn, f"dense layer stage, {dtype}")


def test_fft_layer_operations():
    L = fft_inputs.conv_layer(8, 12, 20, 32, 7, seed=3)
    x, w, g = to_dev(L.x), to_dev(L.w), to_dev(L.g)
    buf = fft.FrequencyBuffer()
    fft.fprop(x, w, buf)  # size the frequency buffer before capture

    def fn():
        return [fft.fprop(x, w, buf), fft.bprop(g, w, L.n, buf), fft.accgrad(x, g, L.k, buf)]

    _capture_and_check(fn, "FFT convolution layer operations")
