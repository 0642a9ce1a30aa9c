"""GPU parity of the shared-buffer DenseNet layer stage (include/dense_bn.h)
against the binary64 oracle (oracle/dense_oracle.py).

README of efficient_densenet_pytorch, "A memory-efficient implementation of
DenseNets", Motivation: concatenation + batch normalization + ReLU, written
to a shared buffer and recomputed in the backward.

Rules (oracle/compare.py), rtol = 1e-5 against the oracle's term scale:
z and dx in binary32 within 1e-5 of the term size, in bfloat16 within one
step or within 1e-5 of the term size; dgamma and dbeta (binary32) the same;
statistics (binary64) to 1e-12.  Cases: ragged and element-wise paths
(hw = 49, 1), vector paths (hw = 64, 1024), DenseNet-BC-100 layers at full
size, 64 and 70 sources, constant channels, gamma of both signs and zero,
a single element per channel, misaligned views, determinism.
"""

import numpy as np
import pytest
import torch

from memory_efficient_activation_amd import dense, dense_inputs as di, inputs
from oracle import dense_oracle as do
from oracle.compare import bf16_scaled_report, f32_report

from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu

RTOL = 1e-5


def _values(a):
    return inputs.decode(a).astype(np.float64)


def _cmp(got, want64, scale, dtype, oracle):
    if dtype == "bf16":
        return bf16_scaled_report(got, oracle.round_array(want64, "bf16"), want64, scale, RTOL)
    return f32_report(got, oracle.round_array(want64, "f32"), scale, RTOL)


def run_layer(w: di.DenseLayer, oracle, label="", src_views=None):
    """Stats, forward and backward of layer w on the GPU, each checked
    against the oracle.  Returns the reports."""
    xs = src_views if src_views is not None else [to_dev(s) for s in w.sources]
    gamma, beta = to_dev(w.gamma), to_dev(w.beta)
    dz = to_dev(w.dz)
    stats = [dense.bn_stats(x) for x in xs]
    z = dense.bn_relu_fwd(xs, stats, gamma, beta, w.eps)
    dxs, dg, db = dense.bn_relu_bwd(xs, stats, gamma, beta, dz, w.eps)
    torch.cuda.synchronize()

    srcs = [_values(s) for s in w.sources]
    zo, f = do.forward(srcs, w.gamma, w.beta, w.eps)
    duo, dgo, dbo, aux = do.backward(srcs, _values(w.dz), w.gamma, w.beta, w.eps)
    rep = {}
    # Statistics.
    mean = np.concatenate([to_host(s)[:, 0] for s in stats])
    var = np.concatenate([to_host(s)[:, 1] for s in stats])
    size = np.abs(f["mean"]) + np.sqrt(f["var"])
    rep["stats"] = {"mean_err": float((np.abs(mean - f["mean"]) / size).max()),
                    "var_err": float((np.abs(var - f["var"]) / np.maximum(f["var"], 1e-300)).max())}
    assert rep["stats"]["mean_err"] <= 1e-12 and rep["stats"]["var_err"] <= 1e-10, rep["stats"]
    rep["z"] = _cmp(to_host(z), zo, f["scale"], w.dtype, oracle)
    assert rep["z"]["ok"], (label, "z", rep["z"])
    for j, dx in enumerate(dxs):
        r = _cmp(to_host(dx), duo[j], aux["du_scale"][j], w.dtype, oracle)
        assert r["ok"], (label, "dx", j, r)
        rep.setdefault("dx", []).append(r)
    rep["dgamma"] = f32_report(to_host(dg), dgo.astype(np.float32), aux["dgamma_scale"], RTOL)
    rep["dbeta"] = f32_report(to_host(db), dbo.astype(np.float32), aux["dbeta_scale"], RTOL)
    assert rep["dgamma"]["ok"] and rep["dbeta"]["ok"], (label, rep["dgamma"], rep["dbeta"])
    if label:
        worst = max((r.get("max_rel", r.get("max_ulp", 0)) for r in rep["dx"]), default=0)
        say(f"[dense] {label}: stats {rep['stats']}, z {_brief(rep['z'])}, dx worst {worst}, "
            f"dgamma {rep['dgamma']['max_rel']:.2e}, dbeta {rep['dbeta']['max_rel']:.2e}")
    return rep, (z, dxs, dg, db, stats)


def _brief(r):
    return {k: v for k, v in r.items() if k in ("max_rel", "max_ulp", "n_off_by_one",
                                                 "n_beyond_one_within_scale", "n_bad")}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chans,n,hw", [([3, 5, 1], 3, 49), ([2, 7], 5, 64), ([4], 1, 1),
                                        ([6, 2], 2, 1), ([5, 3], 4, 1024), ([1, 1, 1], 7, 585)])
def test_small_layers(chans, n, hw, dtype, oracle):
    w = di.dense_layer(chans, n, hw, dtype, seed=sum(chans) + n + hw)
    run_layer(w, oracle, f"{chans} n={n} hw={hw} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("block", [0, 1, 2])
def test_densenet_bc100_last_layer_of_each_block(block, dtype, oracle):
    """The widest layer of each dense block of DenseNet-BC-100 at batch 64."""
    w = di.densenet_bc100_layer(block, di.BLOCK_LAYERS - 1, dtype)
    run_layer(w, oracle, w.name)


def test_ragged_chunk_and_many_sources(oracle):
    """n hw = 4097 (one element past a chunk), 70 sources (two calls)."""
    w = di.dense_layer([1] * 70, 17, 241, "f32", seed=3)
    run_layer(w, oracle, "70 sources, n hw = 4097")
    w = di.dense_layer([2] * 64, 3, 40, "bf16", seed=4)
    run_layer(w, oracle, "64 sources bf16")


def test_special_channels(oracle):
    """Constant channels (variance 0), gamma < 0, gamma = 0 with beta of
    both signs, beta far above and below the normalized values."""
    w = di.dense_layer([6, 3], 4, 96, "f32", seed=5)
    w.sources[0][:, 0, :] = 1.5            # constant channel, beta > 0 below
    w.sources[0][:, 1, :] = -2.25          # constant channel, beta < 0 below
    w.gamma[:] = [1.0, 1.0, -0.75, 0.0, 0.0, 2.0, -1.25, 1.0, 0.5]
    w.beta[:] = [0.5, -0.5, 0.25, 0.75, -0.75, 50.0, -60.0, 0.0, 0.0]
    run_layer(w, oracle, "special channels f32")
    wb = di.dense_layer([6, 3], 4, 96, "bf16", seed=5)
    wb.sources[0][:, 0, :] = inputs.encode(np.full((4, 96), 1.5), "bf16")
    wb.gamma[:] = w.gamma
    wb.beta[:] = w.beta
    run_layer(wb, oracle, "special channels bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_misaligned_views_take_the_element_path(dtype, oracle):
    """Sources that are views at odd element offsets (16-byte vectors do not
    fit): same results through the element-wise kernels."""
    w = di.dense_layer([3, 2], 2, 64, dtype, seed=6)
    views = []
    for s in w.sources:
        flat = np.concatenate([s.ravel()[:1], s.ravel()])
        t = to_dev(flat)[1:].view(s.shape)
        assert t.data_ptr() % 16 != 0
        views.append(t)
    run_layer(w, oracle, f"misaligned views {dtype}", src_views=views)


def test_deterministic_and_shared_buffer_reuse(oracle):
    w = di.densenet_bc100_layer(0, 7, "bf16", n=16)
    _, a = run_layer(w, oracle)
    _, b = run_layer(w, oracle)
    for u, v in zip(a[1] + [a[0], a[2], a[3]], b[1] + [b[0], b[2], b[3]]):
        assert torch.equal(u.view(torch.uint8) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.uint8) if v.dtype == torch.bfloat16 else v)
    # Writing into a shared buffer gives the same bits as a fresh output.
    xs = [to_dev(s) for s in w.sources]
    stats = [dense.bn_stats(x) for x in xs]
    buf = dense.SharedBuffer()
    big = buf.view((16, 400, 32, 32), torch.bfloat16, "cuda")
    big.fill_(7.0)
    z = buf.view(a[0].shape, torch.bfloat16, "cuda")
    dense.bn_relu_fwd(xs, stats, to_dev(w.gamma), to_dev(w.beta), w.eps, out=z)
    torch.cuda.synchronize()
    assert torch.equal(z.view(torch.int16), a[0].view(torch.int16))


def test_bottleneck_stage_autograd_matches_plain_pytorch():
    """EfficientBottleneckStage (shared buffer, recompute) against the plain
    cat -> batch_norm -> relu -> conv stage: same output and gradients in
    binary32."""
    torch.manual_seed(0)
    shared = dense.SharedBuffer()
    eff = dense.EfficientBottleneckStage(60, 48, shared).cuda()
    nai = dense.NaiveBottleneckStage(60, 48).cuda()
    with torch.no_grad():
        nai.weight.copy_(eff.weight)
        eff.gamma.copy_(1 + 0.2 * torch.randn(60))
        eff.beta.copy_(0.3 * torch.randn(60))
        nai.gamma.copy_(eff.gamma)
        nai.beta.copy_(eff.beta)
    xs = [torch.randn(8, c, 16, 16, device="cuda") * 1.5 + 0.5 for c in (24, 12, 12, 12)]
    xa = [x.clone().requires_grad_(True) for x in xs]
    xb = [x.clone().requires_grad_(True) for x in xs]
    stats = [dense.bn_stats(x) for x in xa]
    ya = eff(xa, stats)
    yb = nai(xb)
    r = torch.randn_like(ya)
    (ya * r).sum().backward()
    (yb * r).sum().backward()
    torch.cuda.synchronize()

    def rel(a, b):
        return float((a - b).abs().max() / b.abs().max())

    assert rel(ya, yb) < 1e-5
    for a, b in zip(xa, xb):
        assert rel(a.grad, b.grad) < 1e-4
    assert rel(eff.gamma.grad, nai.gamma.grad) < 1e-4
    assert rel(eff.beta.grad, nai.beta.grad) < 1e-4
    assert rel(eff.weight.grad, nai.weight.grad) < 1e-4
    say(f"[dense] bottleneck autograd: out {rel(ya, yb):.2e}, dx "
        f"{max(rel(a.grad, b.grad) for a, b in zip(xa, xb)):.2e}, dgamma "
        f"{rel(eff.gamma.grad, nai.gamma.grad):.2e}, dW {rel(eff.weight.grad, nai.weight.grad):.2e}")


def test_errors_with_device_buffers():
    x = torch.randn(2, 4, 8, device="cuda")
    st = dense.bn_stats(x)
    g = torch.ones(4, device="cuda")
    b = torch.zeros(4, device="cuda")
    with pytest.raises(ValueError):
        dense.bn_relu_fwd([x], [st], g[:3], b[:3])
    with pytest.raises(ValueError):
        dense.bn_relu_fwd([x], [st.float()], g, b)
    with pytest.raises(RuntimeError):
        dense.bn_relu_fwd([x.cpu()], [st], g, b)
    z = torch.empty(2, 4, 8, device="cuda")
    from memory_efficient_activation_amd import _lib
    # The shared buffer may not overlap a source.
    with pytest.raises(_lib.MeswishError) as e:
        dense.bn_relu_fwd([x], [st], g, b, out=x)
    assert e.value.status == _lib.EALIAS
    dense.bn_relu_fwd([x], [st], g, b, out=z)
    torch.cuda.synchronize()
