"""The DenseNet layer stage's backward without a workspace argument
(dense_bn_relu_bwd_noalloc, for callers that cannot allocate device memory)
against the entry point that takes one (dense_bn_relu_bwd), through the C
ABI: bit for bit, on two calls in a row, the second with a smaller input,
so that the static array keeps the first call's partial sums when the
second starts.  Both are also held to the oracle's rule, and a call that
needs more than the static array holds is refused before any launch."""

import ctypes

import numpy as np
import pytest
import torch

from memory_efficient_activation_amd import _lib, dense, dense_inputs as di, inputs
from oracle import dense_oracle as do
from oracle.compare import bf16_scaled_report, f32_report

from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _descs(xs, dxs, stats, channels):
    offs = np.concatenate([[0], np.cumsum(channels)[:-1]]).astype(int)
    return (_lib.DenseSource * len(xs))(*[
        _lib.DenseSource(x.data_ptr(), d.data_ptr(), s.data_ptr(), int(c), int(o))
        for x, d, s, c, o in zip(xs, dxs, stats, channels, offs)])


def _backward(lib, w, noalloc):
    """One backward of layer w through the C ABI; returns host copies of
    (dxs, dgamma, dbeta)."""
    dev = torch.device("cuda:0")
    xs = [to_dev(s) for s in w.sources]
    stats = [dense.bn_stats(x) for x in xs]
    gamma, beta, dz = to_dev(w.gamma), to_dev(w.beta), to_dev(w.dz)
    C = sum(w.channels)
    dxs = [torch.full_like(x, float("nan")) for x in xs]
    dg = torch.full((C,), float("nan"), dtype=torch.float32, device=dev)
    db = torch.full((C,), float("nan"), dtype=torch.float32, device=dev)
    src = _descs(xs, dxs, stats, w.channels)
    code = _lib.F32 if w.dtype == "f32" else _lib.BF16
    sh = torch.cuda.current_stream(dev).cuda_stream
    if noalloc:
        st = lib.dense_bn_relu_bwd_noalloc(src, len(xs), w.n, w.hw, C, gamma.data_ptr(),
                                           beta.data_ptr(), w.eps, dz.data_ptr(), dg.data_ptr(),
                                           db.data_ptr(), code, sh)
    else:
        nb = lib.dense_bn_workspace_bytes(w.n, C, w.hw)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        st = lib.dense_bn_relu_bwd(src, len(xs), w.n, w.hw, C, gamma.data_ptr(), beta.data_ptr(),
                                   w.eps, dz.data_ptr(), dg.data_ptr(), db.data_ptr(),
                                   ws.data_ptr(), nb, code, sh)
    _lib.check(st, "dense backward")
    torch.cuda.synchronize()
    return [to_host(d) for d in dxs], to_host(dg), to_host(db)


def _oracle_ok(w, got, oracle):
    srcs = [inputs.decode(s).astype(np.float64) for s in w.sources]
    duo, dgo, dbo, aux = do.backward(srcs, inputs.decode(w.dz).astype(np.float64), w.gamma,
                                     w.beta, w.eps)
    dxs, dg, db = got
    for j, dx in enumerate(dxs):
        if w.dtype == "bf16":
            r = bf16_scaled_report(dx, oracle.round_array(duo[j], "bf16"), duo[j],
                                   aux["du_scale"][j])
        else:
            r = f32_report(dx, oracle.round_array(duo[j], "f32"), aux["du_scale"][j])
        assert r["ok"], (w.name, j, r)
    assert f32_report(dg, dgo.astype(np.float32), aux["dgamma_scale"])["ok"]
    assert f32_report(db, dbo.astype(np.float32), aux["dbeta_scale"])["ok"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_backward_equals_the_workspace_backward(dtype, oracle):
    lib = _lib.library()
    # A DenseNet-BC-100 layer (204 channels of 64 x 32 x 32: 52 KiB of
    # partial sums), then a smaller ragged one: the second call reads only
    # slots it wrote itself.
    big = di.densenet_bc100_layer(0, di.BLOCK_LAYERS - 1, dtype)
    small = di.dense_layer([5, 3, 12], 3, 49, dtype, seed=4, name="small ragged layer")
    for w in (big, small):
        want = _backward(lib, w, noalloc=False)
        got = _backward(lib, w, noalloc=True)
        for j, (a, b) in enumerate(zip(got[0], want[0])):
            assert a.tobytes() == b.tobytes(), (w.name, "dx", j)
        assert got[1].tobytes() == want[1].tobytes(), (w.name, "dgamma")
        assert got[2].tobytes() == want[2].tobytes(), (w.name, "dbeta")
        _oracle_ok(w, got, oracle)
        say(f"[noalloc] {dtype} {w.name}: bitwise equal to the workspace backward, oracle rule ok")


def test_noalloc_refuses_more_than_the_static_array():
    """2048 channels of 2^20 elements need 8 MiB of partial sums, twice the
    array: refused with MESWISH_ESCRATCH before anything is launched (the
    source addresses are never dereferenced on that path)."""
    lib = _lib.library()
    C, n, hw = 2048, 1024, 1024
    need = lib.dense_bn_workspace_bytes(n, C, hw)
    assert need > _lib.DENSE_STATIC_WORKSPACE_BYTES
    dev = torch.device("cuda:0")
    small = torch.zeros(64, dtype=torch.float32, device=dev)
    base = 1 << 44  # distinct, never-dereferenced addresses for the size checks
    src = (_lib.DenseSource * 1)(_lib.DenseSource(base, base + (1 << 40), small.data_ptr(), C, 0))
    stats = torch.zeros((C, 2), dtype=torch.float64, device=dev)
    src[0].stats = stats.data_ptr()
    p = torch.zeros(4 * C, dtype=torch.float32, device=dev)
    st = lib.dense_bn_relu_bwd_noalloc(src, 1, n, hw, C, p[:C].data_ptr(), p[C:2 * C].data_ptr(),
                                       1e-5, base + (2 << 40), p[2 * C:3 * C].data_ptr(),
                                       p[3 * C:].data_ptr(), _lib.F32,
                                       torch.cuda.current_stream(dev).cuda_stream)
    assert st == _lib.ESCRATCH
    assert b"static" in lib.meswish_strerror(st)
    torch.cuda.synchronize()
