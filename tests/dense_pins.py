"""Pins of the DenseNet-layer oracle (oracle/dense_oracle.py).

Each ``pin_*`` takes the oracle module ``d`` and raises AssertionError when
the oracle disagrees with a fact that does not come from the oracle itself:

* binary64 PyTorch CPU autograd of torch.cat + torch's batch_norm (training
  mode) + relu -- an independent implementation of the same layer stage;
* closed forms: a constant channel (variance 0, so xhat = 0 and
  z = ReLU(beta)); a channel of two values a, b (xhat = +-d / sqrt(d^2 + eps)
  with d = (a - b) / 2);
* invariants of batch normalization's backward: the input gradient of each
  channel sums to 0, and its dot product with xhat equals
  gamma r sum(g xhat) eps / (var + eps);
* mean and variance of the output where the ReLU passes everything;
* central finite differences of a weighted sum of z;
* channel independence: concatenation does not mix channels, so the layer
  over [A, B] equals the layers over [A] and [B] side by side;
* equivariance under a permutation of the batch.

``tests/test_dense_oracle.py`` runs them, and plants mistakes in a copy of
the oracle to check that each is caught by at least one pin.
"""

from __future__ import annotations

import numpy as np

EPS = 1e-5


def _case(seed, channels=(3, 5, 2), n=4, p=6, gamma_scale=0.3):
    rng = np.random.default_rng(seed)
    srcs = [rng.standard_normal(c)[None, :, None] + rng.uniform(0.5, 2, c)[None, :, None]
            * rng.standard_normal((n, c, p)) for c in channels]
    total = sum(channels)
    gamma = 1 + gamma_scale * rng.standard_normal(total)
    beta = 0.5 * rng.standard_normal(total)
    dz = rng.standard_normal((n, total, p))
    return srcs, gamma, beta, dz


def pin_torch_autograd(d):
    import torch
    import torch.nn.functional as F
    for seed, chans, n, p in ((1, (3, 5, 2), 4, 6), (2, (1, 7), 3, 11), (3, (4,), 2, 1), (4, (2, 2, 2, 2), 1, 9)):
        srcs, gamma, beta, dz = _case(seed, chans, n, p)
        ts = [torch.tensor(s, dtype=torch.float64, requires_grad=True) for s in srcs]
        tg = torch.tensor(gamma, dtype=torch.float64, requires_grad=True)
        tb = torch.tensor(beta, dtype=torch.float64, requires_grad=True)
        u = torch.cat(ts, dim=1)
        z = torch.relu(F.batch_norm(u, None, None, tg, tb, training=True, eps=EPS))
        z.backward(torch.tensor(dz, dtype=torch.float64))
        zo, f = d.forward(srcs, gamma, beta, EPS)
        assert np.allclose(zo, z.detach().numpy(), rtol=0, atol=1e-13 * (1 + np.abs(zo).max()))
        dus, dg, db, aux = d.backward(srcs, dz, gamma, beta, EPS)
        for j, t in enumerate(ts):
            m = aux["du_scale"][j]
            err = np.abs(dus[j] - t.grad.numpy())
            assert np.all(err <= 1e-12 * m + 1e-300), (seed, j, err.max())
        assert np.all(np.abs(dg - tg.grad.numpy()) <= 1e-12 * aux["dgamma_scale"] + 1e-300)
        assert np.all(np.abs(db - tb.grad.numpy()) <= 1e-12 * aux["dbeta_scale"] + 1e-300)


def _torch_layer(srcs, gamma, beta, dz):
    """binary64 PyTorch CPU: z, and the gradients of the sources, gamma and
    beta, by autograd of torch.cat + batch_norm (training) + relu."""
    import torch
    import torch.nn.functional as F
    ts = [torch.tensor(s, dtype=torch.float64, requires_grad=True) for s in srcs]
    tg = torch.tensor(gamma, dtype=torch.float64, requires_grad=True)
    tb = torch.tensor(beta, dtype=torch.float64, requires_grad=True)
    z = torch.relu(F.batch_norm(torch.cat(ts, dim=1), None, None, tg, tb, training=True, eps=EPS))
    z.backward(torch.tensor(dz, dtype=torch.float64))
    return (z.detach().numpy(), [t.grad.numpy() for t in ts], tg.grad.numpy(), tb.grad.numpy())


def pin_scales_attained(d):
    """Each error scale is the sum of the absolute values of the terms its
    result sums, so it equals |result| where all terms share a sign: the
    scales are tight, not merely upper bounds (an inflated scale would
    loosen the tolerance it sets).  One channel, values by hand, results
    from PyTorch autograd:
      forward: gamma > 0, beta > 0, mean < 0, u > 0    -> z = scale;
      dbeta: every g > 0 (beta large: ReLU passes all) -> dbeta = scale;
      dgamma: mean exactly 0, g with the sign of u     -> dgamma = scale;
      du at element e: mean 0, g_e > 0, dbeta < 0 and u_e dgamma < 0, so
        gamma r g_e, -gamma r dbeta / M and -gamma r xhat_e dgamma / M are
        all positive                                    -> du_e = scale_e."""
    # Forward: mean = -1.25 < 0; elements 3..5 have u > 0.
    u = np.array([-5.0, -4.0, -3.0, 1.0, 2.0, 1.5])[None, None, :]
    gamma, beta = np.array([0.7]), np.array([0.3])
    dz = np.ones_like(u)
    z, aux = d.forward([u], gamma, beta, EPS)
    zt = _torch_layer([u], gamma, beta, dz)[0]
    pos = u > 0
    assert np.allclose(aux["scale"][pos], zt[pos], rtol=1e-13, atol=0), (aux["scale"][pos], zt[pos])
    # Backward: symmetric values (mean exactly 0), beta large.
    u = np.array([-3.0, -1.0, 1.0, 3.0])[None, None, :]
    gamma, beta = np.array([0.5]), np.array([10.0])
    for dz, what in ((np.array([0.5, 1.5, 2.0, 0.7]), "dbeta"),
                     (np.array([-0.5, -1.5, 2.0, 0.7]), "dgamma"),
                     (np.array([1.0, -0.5, 0.2, -1.5]), "du")):
        dz = dz[None, None, :]
        _, dut, dgt, dbt = _torch_layer([u], gamma, beta, dz)
        dus, dg, db, aux = d.backward([u], dz, gamma, beta, EPS)
        if what == "dbeta":
            assert np.allclose(aux["dbeta_scale"], np.abs(dbt), rtol=1e-13, atol=0)
        elif what == "dgamma":
            assert np.allclose(aux["dgamma_scale"], np.abs(dgt), rtol=1e-13, atol=0)
        else:
            assert dbt[0] < 0 and dgt[0] < 0  # the sign conditions of element e = 2
            e = (0, 0, 2)
            assert np.isclose(aux["du_scale"][0][e], abs(dut[0][e]), rtol=1e-13, atol=0), \
                (aux["du_scale"][0][e], dut[0][e])
        # Everywhere, the scales bound the results.
        assert np.all(np.abs(dut[0]) <= aux["du_scale"][0] * (1 + 1e-13))
        assert np.all(np.abs(dgt) <= aux["dgamma_scale"] * (1 + 1e-13))
        assert np.all(np.abs(dbt) <= aux["dbeta_scale"] * (1 + 1e-13))


def pin_constant_channel(d):
    """Variance 0: xhat = 0, z = ReLU(beta); du = gamma / sqrt(eps) (g - mean g)."""
    srcs, gamma, beta, dz = _case(5, (3,), 4, 5)
    srcs[0][:, 1, :] = 2.75
    beta[1] = 0.5
    z, f = d.forward(srcs, gamma, beta, EPS)
    assert f["var"][1] == 0.0 and f["mean"][1] == 2.75
    assert np.all(z[:, 1, :] == 0.5)
    dus, dg, db, _ = d.backward(srcs, dz, gamma, beta, EPS)
    g = dz[:, 1, :]
    want = gamma[1] / np.sqrt(EPS) * (g - g.mean())
    assert np.allclose(dus[0][:, 1, :], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    assert dg[1] == 0.0 and np.isclose(db[1], g.sum(), rtol=1e-14)
    beta[1] = -0.5  # ReLU closes: nothing passes
    z, _ = d.forward(srcs, gamma, beta, EPS)
    assert np.all(z[:, 1, :] == 0.0)
    dus, dg, db, _ = d.backward(srcs, dz, gamma, beta, EPS)
    assert np.all(dus[0][:, 1, :] == 0.0) and db[1] == 0.0


def pin_two_values(d):
    """A channel holding a and b (N P = 2): mean (a + b) / 2, variance d^2,
    xhat = +-d / sqrt(d^2 + eps), d = (a - b) / 2."""
    a, b = 1.75, -0.5
    src = np.array([[[a, b]]])
    for gamma, beta in ((2.0, 0.25), (-1.5, 3.0), (0.5, -4.0)):
        z, f = d.forward([src], [gamma], [beta], EPS)
        dd = (a - b) / 2
        xh = dd / np.sqrt(dd * dd + EPS)
        assert np.isclose(f["mean"][0], (a + b) / 2, rtol=1e-15)
        assert np.isclose(f["var"][0], dd * dd, rtol=1e-15)
        want = np.maximum([gamma * xh + beta, -gamma * xh + beta], 0.0)
        assert np.allclose(z.ravel(), want, rtol=1e-14, atol=1e-15)


def pin_backward_invariants(d):
    for seed in range(6, 10):
        srcs, gamma, beta, dz = _case(seed, (4, 3), 5, 7)
        dus, dg, db, aux = d.backward(srcs, dz, gamma, beta, EPS)
        du = np.concatenate(dus, axis=1)
        _, f = d.forward(srcs, gamma, beta, EPS)
        m = aux["du_scale"]
        scale = np.concatenate(m, axis=1).sum(axis=(0, 2))
        assert np.all(np.abs(du.sum(axis=(0, 2))) <= 1e-13 * scale)
        r = 1 / np.sqrt(f["var"] + EPS)
        g = np.where(f["h"] > 0, dz, 0.0)
        want = gamma * r * (g * f["xhat"]).sum(axis=(0, 2)) * EPS / (f["var"] + EPS)
        got = (du * f["xhat"]).sum(axis=(0, 2))
        assert np.all(np.abs(got - want) <= 1e-12 * (scale * np.abs(f["xhat"]).max())), seed


def pin_output_moments(d):
    """With beta far above gamma xhat the ReLU passes everything: each
    channel of z has mean beta and variance gamma^2 var / (var + eps)."""
    srcs, gamma, beta, _ = _case(11, (3, 4), 6, 8)
    beta = beta + 100.0
    z, f = d.forward(srcs, gamma, beta, EPS)
    assert np.allclose(z.mean(axis=(0, 2)), beta, rtol=1e-14)
    want = gamma ** 2 * f["var"] / (f["var"] + EPS)
    assert np.allclose(z.var(axis=(0, 2)), want, rtol=1e-9)


def pin_finite_differences(d):
    srcs, gamma, beta, _ = _case(13, (2, 3), 3, 4)
    rng = np.random.default_rng(14)
    w = rng.standard_normal((3, 5, 4))
    loss = lambda s, g, b: float((d.forward(s, g, b, EPS)[0] * w).sum())
    dus, dg, db, _ = d.backward(srcs, w, gamma, beta, EPS)
    h = 1e-6
    for j, s in enumerate(srcs):
        for idx in [(0, 0, 0), (2, s.shape[1] - 1, 3), (1, 0, 2)]:
            sp = [t.copy() for t in srcs]
            sm = [t.copy() for t in srcs]
            sp[j][idx] += h
            sm[j][idx] -= h
            fd = (loss(sp, gamma, beta) - loss(sm, gamma, beta)) / (2 * h)
            assert abs(fd - dus[j][idx]) <= 1e-6 * (1 + abs(fd)), (j, idx, fd, dus[j][idx])
    for c in range(5):
        gp, gm = gamma.copy(), gamma.copy()
        gp[c] += h
        gm[c] -= h
        fd = (loss(srcs, gp, beta) - loss(srcs, gm, beta)) / (2 * h)
        assert abs(fd - dg[c]) <= 1e-6 * (1 + abs(fd)), c
        bp, bm = beta.copy(), beta.copy()
        bp[c] += h
        bm[c] -= h
        fd = (loss(srcs, gamma, bp) - loss(srcs, gamma, bm)) / (2 * h)
        assert abs(fd - db[c]) <= 1e-6 * (1 + abs(fd)), c


def pin_channel_independence(d):
    srcs, gamma, beta, dz = _case(17, (3, 4, 2), 3, 5)
    z, _ = d.forward(srcs, gamma, beta, EPS)
    dus, dg, db, _ = d.backward(srcs, dz, gamma, beta, EPS)
    c0 = 0
    for j, s in enumerate(srcs):
        c = s.shape[1]
        sl = slice(c0, c0 + c)
        zj, _ = d.forward([s], gamma[sl], beta[sl], EPS)
        assert np.array_equal(zj, z[:, sl, :])
        duj, dgj, dbj, _ = d.backward([s], dz[:, sl, :], gamma[sl], beta[sl], EPS)
        assert np.allclose(duj[0], dus[j], rtol=1e-13, atol=1e-15)
        assert np.allclose(dgj, dg[sl], rtol=1e-13) and np.allclose(dbj, db[sl], rtol=1e-13)
        c0 += c


def pin_batch_permutation(d):
    srcs, gamma, beta, dz = _case(19, (2, 3), 5, 4)
    perm = np.array([3, 0, 4, 2, 1])
    z, _ = d.forward(srcs, gamma, beta, EPS)
    zp, _ = d.forward([s[perm] for s in srcs], gamma, beta, EPS)
    assert np.allclose(zp, z[perm], rtol=1e-13, atol=1e-15)
    dus, _, _, _ = d.backward(srcs, dz, gamma, beta, EPS)
    dup, _, _, _ = d.backward([s[perm] for s in srcs], dz[perm], gamma, beta, EPS)
    for a, b in zip(dus, dup):
        assert np.allclose(b, a[perm], rtol=1e-12, atol=1e-14)


ALL_PINS = [pin_torch_autograd, pin_scales_attained, pin_constant_channel, pin_two_values, pin_backward_invariants,
            pin_output_moments, pin_finite_differences, pin_channel_independence,
            pin_batch_permutation]
