"""GPU parity of the FFT convolution layers (include/fft_conv.h) against the
binary64 oracle (oracle/fft_oracle.py).

"Fast Training of Convolutional Networks through FFTs": transforms, per-bin
products, inverse transforms, and the three layer operations built on them.

Rules (reading of the fp32 1e-5 bound for a method whose errors are
normwise): every output map within 1e-5 of the largest magnitude any of
its elements can have --
  spectra:   n ||x||_2            (the transform's 2-norm, Parseval)
  inverse:   sqrt(2) ||Y_half||_2 / n  (bounds every element of the inverse)
  products:  sum_k |a_ik| |b_kj|  (the size of the terms, per element)
  layers:    sum over the paired maps of ||.||_2 ||.||_2  (Cauchy-Schwarz).
Full-size layers are checked on sampled output maps, each computed by the
oracle's direct definition.
"""

import numpy as np
import pytest
import torch

from memory_efficient_activation_amd import fft, fft_inputs
from oracle import fft_oracle as fo_

from gpu_util import say

pytestmark = pytest.mark.gpu
RTOL = 1e-5


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _host(t):
    return t.detach().cpu().numpy()


def _maxrel(err, scale):
    return float((err / np.maximum(scale, 1e-300)).max()) if err.size else 0.0


@pytest.mark.parametrize("n", [8, 16, 32, 64])
@pytest.mark.parametrize("m_kind", ["full", "kernel", "output", "one"])
def test_r2c_matches_the_dft(n, m_kind, oracle):
    m = {"full": n, "kernel": min(7, n), "output": n - min(7, n) + 1, "one": 1}[m_kind]
    B = 3 * (512 // n) + 5  # several blocks and a partial one
    x = np.random.default_rng(n + m).standard_normal((B, m, m)).astype(np.float32)
    spec = _host(fft.r2c(_dev(x), n))                     # [P, B]
    want = fo_.rfft2_half(x, n).reshape(B, -1).T          # [P, B]
    scale = fo_.spectrum_scale(x, n)[None, :]
    r = _maxrel(np.abs(spec - want), scale)
    say(f"[fft] r2c n={n} m={m} B={B}: max err / (n ||x||) = {r:.2e}")
    assert r <= RTOL


@pytest.mark.parametrize("n", [8, 16, 32, 64])
def test_c2r_matches_the_inverse(n):
    B = 2 * (512 // n) + 3
    rng = np.random.default_rng(100 + n)
    x = rng.standard_normal((B, n, n))
    half = fo_.rfft2_half(x, n)
    half = half + 0.1 * (rng.standard_normal(half.shape) + 1j * rng.standard_normal(half.shape))
    spec = half.reshape(B, -1).T.astype(np.complex64)
    for m in (n, n // 2 + 1, 1):
        got = _host(fft.c2r(_dev(spec), n, m, 1.0 / (n * n)))
        want = fo_.irfft2_crop(spec.T.reshape(B, n, n // 2 + 1).astype(np.complex128), n, m)
        scale = np.sqrt(2.0) * np.sqrt((np.abs(spec.astype(np.complex128)) ** 2).sum(0)) / n
        r = _maxrel(np.abs(got - want).reshape(B, -1).max(1), scale)
        say(f"[fft] c2r n={n} m={m}: max err / scale = {r:.2e}")
        assert r <= RTOL


@pytest.mark.parametrize("n,m", [(8, 7), (16, 9), (32, 26), (32, 7), (32, 32)])
def test_inverse_into_an_unaligned_output(n, m, oracle):
    """Outputs need only 4-byte alignment: an inverse written one float past
    a 16-byte boundary takes the element-wise store path and gives the same
    values (the round trip through both transforms), writing nothing outside
    its range.  Inputs must be 16-byte aligned and are rejected otherwise."""
    B = 2 * (512 // n) + 3
    x = np.random.default_rng(7 * n + m).standard_normal((B, m, m)).astype(np.float32)
    spec = fft.r2c(_dev(x), n)
    lib = fft._lib.library()
    out = torch.full((B * m * m + 2,), 7.0, dtype=torch.float32, device="cuda")
    fft._lib.check(lib.fftconv_c2r(spec.data_ptr(), B, n, m, 1.0 / (n * n), out.data_ptr() + 4, None),
                   "fftconv_c2r")
    torch.cuda.synchronize()
    o = _host(out)
    r = float(np.abs(o[1:-1].reshape(B, m, m) - x).max() / np.abs(x).max())
    say(f"[fft] c2r into an output 4 bytes past alignment, n={n} m={m} B={B}: round trip {r:.2e}")
    assert r <= RTOL
    assert o[0] == 7.0 and o[-1] == 7.0
    xs = torch.zeros(B * m * m + 1, dtype=torch.float32, device="cuda")
    assert lib.fftconv_r2c(xs.data_ptr() + 4, B, m, n, spec.data_ptr(), None) == fft._lib.EINVAL


@pytest.mark.parametrize("op", [0, 1, 2])
@pytest.mark.parametrize("S,f,fo,P", [(3, 5, 7, 9), (70, 33, 65, 5), (128, 96, 130, 3)])
def test_cmul_matches_the_per_bin_products(op, S, f, fo, P):
    rng = np.random.default_rng(op * 100 + S)

    def spec(maps):
        return (rng.standard_normal((P, maps)) + 1j * rng.standard_normal((P, maps))).astype(np.complex64)

    a = spec({0: S * f, 1: S * fo, 2: S * fo}[op])
    b = spec({0: fo * f, 1: fo * f, 2: S * f}[op])
    got = _host(fft.cmul(op, _dev(a), _dev(b), S, f, fo))
    A = a.astype(np.complex128).T.reshape({0: (S, f), 1: (S, fo), 2: (S, fo)}[op] + (P, 1))
    Bm = b.astype(np.complex128).T.reshape({0: (fo, f), 1: (fo, f), 2: (S, f)}[op] + (P, 1))
    fun = {0: fo_.freq_fprop, 1: fo_.freq_bprop, 2: fo_.freq_accgrad}[op]
    # The oracle's weight-gradient stage takes (X, G): B holds X, A holds G.
    args = (Bm, A) if op == 2 else (A, Bm)
    want = fun(*args)                                        # [., ., P, 1]
    scale = fun(*(np.abs(t) for t in args)).real             # sum of |terms|
    want = want.reshape(want.shape[0] * want.shape[1], P).T
    scale = scale.reshape(scale.shape[0] * scale.shape[1], P).T
    r = _maxrel(np.abs(got - want), scale)
    say(f"[fft] cmul op={op} S={S} f={f} f'={fo} bins={P}: max err / term size = {r:.2e}")
    assert r <= RTOL


@pytest.mark.parametrize("op", [0, 1, 2])
def test_cmul_operands_off_a_16_byte_boundary(op):
    """The measured layer's shapes with spectra 8 bytes past a 16-byte
    boundary: every tile lies inside the matrices, but the 16-byte pair loads
    need aligned pairs, so the products take the checked loads.  They must
    equal the aligned call's products bit for bit, and the oracle's."""
    S, f, fo, P = 128, 96, 256, 3
    rng = np.random.default_rng(40 + op)
    na, nb = {0: S * f, 1: S * fo, 2: S * fo}[op], {0: fo * f, 1: fo * f, 2: S * f}[op]

    def spec(maps):
        return (rng.standard_normal((P, maps)) + 1j * rng.standard_normal((P, maps))).astype(np.complex64)

    a, b = spec(na), spec(nb)

    def shifted(h):
        buf = torch.empty(h.size + 1, dtype=torch.complex64, device="cuda:0")
        v = buf[1:].view(h.shape)
        v.copy_(torch.from_numpy(h).to("cuda:0"))
        assert v.data_ptr() % 16 == 8
        return v

    aligned = fft.cmul(op, _dev(a), _dev(b), S, f, fo)
    off = fft.cmul(op, shifted(a), shifted(b), S, f, fo)
    torch.cuda.synchronize()
    assert torch.equal(torch.view_as_real(aligned), torch.view_as_real(off))
    A = a.astype(np.complex128).T.reshape({0: (S, f), 1: (S, fo), 2: (S, fo)}[op] + (P, 1))
    Bm = b.astype(np.complex128).T.reshape({0: (fo, f), 1: (fo, f), 2: (S, f)}[op] + (P, 1))
    fun = {0: fo_.freq_fprop, 1: fo_.freq_bprop, 2: fo_.freq_accgrad}[op]
    args = (Bm, A) if op == 2 else (A, Bm)
    want = fun(*args)
    scale = fun(*(np.abs(t) for t in args)).real
    want = want.reshape(want.shape[0] * want.shape[1], P).T
    scale = scale.reshape(scale.shape[0] * scale.shape[1], P).T
    r = _maxrel(np.abs(_host(off) - want), scale)
    say(f"[fft] cmul op={op} off 16-byte boundary: bitwise equal to aligned, max err / term size = {r:.2e}")
    assert r <= RTOL


CASES = [(2, 3, 4, 8, 3), (3, 5, 2, 16, 5), (1, 1, 1, 8, 8), (2, 2, 3, 8, 1), (4, 7, 9, 32, 7),
         (2, 3, 5, 64, 13), (5, 17, 33, 16, 3)]


@pytest.mark.parametrize("S,f,fo,n,k", CASES)
def test_layer_operations_match_the_direct_definition(S, f, fo, n, k):
    w_ = fft_inputs.conv_layer(S, f, fo, n, k, seed=S + f + fo + n + k)
    buf = fft.FrequencyBuffer()
    x, w, g = _dev(w_.x), _dev(w_.w), _dev(w_.g)
    y, gx, gw = fft.fprop(x, w, buf), fft.bprop(g, w, n, buf), fft.accgrad(x, g, k, buf)
    torch.cuda.synchronize()
    r1 = _maxrel(np.abs(_host(y) - fo_.fprop_direct(w_.x, w_.w)).max((2, 3)),
                 fo_.fprop_scale(w_.x, w_.w))
    r2 = _maxrel(np.abs(_host(gx) - fo_.bprop_direct(w_.g, w_.w, n)).max((2, 3)),
                 fo_.bprop_scale(w_.g, w_.w))
    r3 = _maxrel(np.abs(_host(gw) - fo_.accgrad_direct(w_.x, w_.g, k)).max((2, 3)),
                 fo_.accgrad_scale(w_.x, w_.g))
    say(f"[fft] layer {w_.name}: fprop {r1:.2e} bprop {r2:.2e} accgrad {r3:.2e}")
    assert max(r1, r2, r3) <= RTOL


def test_bench_layer_at_full_size_on_sampled_maps():
    """S=128, f=96, f'=256, n=32, k=7: each operation on the whole layer,
    16 output maps of each checked against the direct definition."""
    L = fft_inputs.bench_layer()
    buf = fft.FrequencyBuffer()
    x, w, g = _dev(L.x), _dev(L.w), _dev(L.g)
    y, gx, gw = fft.fprop(x, w, buf), fft.bprop(g, w, L.n, buf), fft.accgrad(x, g, L.k, buf)
    torch.cuda.synchronize()
    y, gx, gw = _host(y), _host(gx), _host(gw)
    rng = np.random.default_rng(42)
    worst = [0.0, 0.0, 0.0]
    for _ in range(16):
        s, fi, oi = rng.integers(L.S), rng.integers(L.f), rng.integers(L.fo)
        want = fo_.fprop_direct(L.x[s:s + 1], L.w[oi:oi + 1])[0, 0]
        sc = fo_.fprop_scale(L.x[s:s + 1], L.w[oi:oi + 1])[0, 0]
        worst[0] = max(worst[0], np.abs(y[s, oi] - want).max() / sc)
        want = fo_.bprop_direct(L.g[s:s + 1], L.w[:, fi:fi + 1], L.n)[0, 0]
        sc = fo_.bprop_scale(L.g[s:s + 1], L.w[:, fi:fi + 1])[0, 0]
        worst[1] = max(worst[1], np.abs(gx[s, fi] - want).max() / sc)
        want = fo_.accgrad_direct(L.x[:, fi:fi + 1], L.g[:, oi:oi + 1], L.k)[0, 0]
        sc = fo_.accgrad_scale(L.x[:, fi:fi + 1], L.g[:, oi:oi + 1])[0, 0]
        worst[2] = max(worst[2], np.abs(gw[oi, fi] - want).max() / sc)
    say(f"[fft] bench layer {L.name}, 16 sampled maps each: fprop {worst[0]:.2e} "
        f"bprop {worst[1]:.2e} accgrad {worst[2]:.2e}")
    assert max(worst) <= RTOL
    assert buf.nbytes == fft._lib.library().fftconv_buffer_bytes(L.S, L.f, L.fo, L.n)


@pytest.mark.parametrize("S,f,fo,n,k", [(16, 32, 48, 64, 9), (64, 48, 80, 16, 5)])
def test_larger_layers_on_sampled_maps(S, f, fo, n, k):
    """n = 64 and n = 16 at sizes that span many blocks of every kernel
    (and 64- and 32-column product tiles): 8 sampled output maps of each
    operation against the direct definition."""
    L = fft_inputs.conv_layer(S, f, fo, n, k, seed=7 * n + k)
    buf = fft.FrequencyBuffer()
    x, w, g = _dev(L.x), _dev(L.w), _dev(L.g)
    y, gx, gw = fft.fprop(x, w, buf), fft.bprop(g, w, n, buf), fft.accgrad(x, g, k, buf)
    torch.cuda.synchronize()
    y, gx, gw = _host(y), _host(gx), _host(gw)
    rng = np.random.default_rng(n)
    worst = [0.0, 0.0, 0.0]
    for _ in range(8):
        s, fi, oi = rng.integers(S), rng.integers(f), rng.integers(fo)
        want = fo_.fprop_direct(L.x[s:s + 1], L.w[oi:oi + 1])[0, 0]
        worst[0] = max(worst[0], np.abs(y[s, oi] - want).max()
                       / fo_.fprop_scale(L.x[s:s + 1], L.w[oi:oi + 1])[0, 0])
        want = fo_.bprop_direct(L.g[s:s + 1], L.w[:, fi:fi + 1], n)[0, 0]
        worst[1] = max(worst[1], np.abs(gx[s, fi] - want).max()
                       / fo_.bprop_scale(L.g[s:s + 1], L.w[:, fi:fi + 1])[0, 0])
        want = fo_.accgrad_direct(L.x[:, fi:fi + 1], L.g[:, oi:oi + 1], k)[0, 0]
        worst[2] = max(worst[2], np.abs(gw[oi, fi] - want).max()
                       / fo_.accgrad_scale(L.x[:, fi:fi + 1], L.g[:, oi:oi + 1])[0, 0])
    say(f"[fft] layer {L.name}, 8 sampled maps each: fprop {worst[0]:.2e} bprop {worst[1]:.2e} "
        f"accgrad {worst[2]:.2e}")
    assert max(worst) <= RTOL


def test_module_autograd_matches_torch_conv2d():
    torch.manual_seed(0)
    buf = fft.FrequencyBuffer()
    m1 = fft.FFTConv2d(6, 10, 9, buf).cuda()        # 16 x 16 -> 8 x 8
    m2 = fft.FFTConv2d(10, 4, 3, buf).cuda()        # 8 x 8 -> 6 x 6, shares the buffer
    x = torch.randn(3, 6, 16, 16, device="cuda", requires_grad=True)
    y = m2(torch.relu(m1(x)))
    r = torch.randn_like(y)
    (y * r).sum().backward()
    torch.cuda.synchronize()
    xr = x.detach().double().cpu().requires_grad_(True)
    w1 = m1.weight.detach().double().cpu().requires_grad_(True)
    w2 = m2.weight.detach().double().cpu().requires_grad_(True)
    yr = torch.nn.functional.conv2d(torch.relu(torch.nn.functional.conv2d(xr, w1)), w2)
    (yr * r.double().cpu()).sum().backward()

    def rel(a, b):
        return float((a.detach().double().cpu() - b).abs().max() / b.abs().max())

    errs = (rel(y, yr.detach()), rel(x.grad, xr.grad), rel(m1.weight.grad, w1.grad),
            rel(m2.weight.grad, w2.grad))
    say(f"[fft] module autograd vs torch conv2d (binary64): y {errs[0]:.2e} dx {errs[1]:.2e} "
        f"dw1 {errs[2]:.2e} dw2 {errs[3]:.2e}")
    assert max(errs) < 1e-5
    # One buffer serves both layers: sized by the larger one.
    lib = fft._lib.library()
    assert buf.nbytes == max(lib.fftconv_buffer_bytes(3, 6, 10, 16), lib.fftconv_buffer_bytes(3, 10, 4, 8))


def test_errors_with_device_buffers():
    from memory_efficient_activation_amd import _lib
    x = torch.randn(2, 3, 12, 12, device="cuda")
    w = torch.randn(4, 3, 3, 3, device="cuda")
    with pytest.raises(ValueError):
        fft.fprop(x, w)                        # n = 12 is not supported
    x = torch.randn(2, 3, 16, 16, device="cuda")
    with pytest.raises(TypeError):
        fft.fprop(x.double(), w.double())
    with pytest.raises(RuntimeError):
        fft.fprop(x.cpu(), w.cpu())
    buf = torch.empty(fft._lib.library().fftconv_buffer_bytes(2, 3, 4, 16), dtype=torch.uint8,
                      device="cuda")
    y = torch.empty(2, 4, 14, 14, device="cuda")
    # Frequency buffer on top of the output.
    st = fft._lib.library().fftconv_fprop(x.data_ptr(), w.data_ptr(), buf.data_ptr(), 2, 3, 4, 16, 3,
                                          buf.data_ptr(), buf.numel(), None)
    assert st == _lib.EALIAS
    assert fft._lib.library().fftconv_fprop(x.data_ptr(), w.data_ptr(), y.data_ptr(), 2, 3, 4, 16, 3,
                                            buf.data_ptr(), buf.numel() - 8, None) == _lib.EINVAL
    torch.cuda.synchronize()
