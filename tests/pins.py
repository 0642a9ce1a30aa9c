"""Checks that pin the CPU oracle to facts that do not come from the oracle.

Each ``pin_*`` function takes an :class:`oracle.Oracle` and raises
``AssertionError`` when the oracle disagrees with:

* the worked numbers and definitions the pages print (golden fixtures under
  ``tests/golden/``, each with its citation);
* closed forms (Lambert-W stationary point, asymptotes, sigma(t)+sigma(-t)=1);
* independent implementations: PyTorch binary64 autograd of the plain module
  from the blog post's "How is Swish implemented?", ``scipy.special.expit``,
  arbitrary-precision evaluation with mpmath, central finite differences;
* exact rational rounding (``fractions.Fraction``) and numpy/torch casts.

``tests/test_oracle_pins.py`` runs them on the real oracle (all must pass);
``tests/test_oracle_mutants.py`` runs them on oracles with planted mistakes
(each mutant must fail at least one).
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _grid(lo, hi, n, seed):
    rng = np.random.default_rng(seed)
    return np.concatenate([np.linspace(lo, hi, n), rng.uniform(lo, hi, n)])


ALPHAS = (1.0, 1.5, 0.5, -1.25)


# --------------------------------------------------------------------------
# Special values and closed forms.
# --------------------------------------------------------------------------

def pin_special_values(o):
    for c in _golden("swish_special_values.json")["cases"]:
        if c["what"].startswith("sigmoid"):
            got = o.sigmoid_f64(c["t"])
        elif c["what"].startswith("swish'"):
            got = o.grad_f64(c["x"], 1.0, c["alpha"])[0]
        else:
            got = o.swish_f64(c["x"], c["alpha"])
        assert got == c["value"], (c, got)


def pin_mpmath_values(o):
    """x * sigma(alpha x) and its derivative at 60 digits (mpmath's own exp)."""
    import mpmath
    mpmath.mp.dps = 60
    for alpha in ALPHAS:
        a = mpmath.mpf(alpha)
        for x in _grid(-60.0, 60.0, 60, 11):
            X = mpmath.mpf(float(x))
            ref_y = X / (1 + mpmath.exp(-a * X))
            ref_g = mpmath.diff(lambda u: u / (1 + mpmath.exp(-a * u)), X)
            y = o.swish_f64(x, alpha)
            g = o.grad_f64(x, 1.0, alpha)[0]
            assert abs(y - float(ref_y)) <= 1e-14 * max(abs(float(ref_y)), 1e-300), (alpha, x, y, ref_y)
            # The derivative sum cancels near its zero: compare against the
            # scale of its terms.
            scale = float(abs(1 / (1 + mpmath.exp(-a * X)))) * (1 + abs(alpha * x))
            assert abs(g - float(ref_g)) <= 1e-14 * max(scale, 1e-300), (alpha, x, g, ref_g)


def pin_sigmoid_vs_expit(o):
    from scipy.special import expit
    for t in _grid(-700.0, 700.0, 2000, 3):
        ref = float(expit(t))
        got = o.sigmoid_f64(t)
        assert abs(got - ref) <= 1e-15 * ref + 1e-320, (t, got, ref)


def pin_odd_part_identity(o):
    """sigma(t) + sigma(-t) = 1 gives y(x) - y(-x) = x and y'(x) + y'(-x) = 1."""
    for alpha in ALPHAS:
        for x in _grid(-30.0, 30.0, 300, 5):
            d = o.swish_f64(x, alpha) - o.swish_f64(-x, alpha)
            assert abs(d - x) <= 1e-15 * max(abs(x), 1.0), (alpha, x, d)
            gsum = o.grad_f64(x, 1.0, alpha)[0] + o.grad_f64(-x, 1.0, alpha)[0]
            assert abs(gsum - 1.0) <= 1e-14 * (1 + abs(alpha * x)), (alpha, x, gsum)


def pin_alpha_scaling(o):
    """Swish_a(x) = Swish_1(a x) / a and Swish_a'(x) = Swish_1'(a x)."""
    for alpha in (1.5, 0.5, -1.25, 3.0):
        for x in _grid(-20.0, 20.0, 200, 7):
            ya = o.swish_f64(x, alpha)
            y1 = o.swish_f64(alpha * x, 1.0) / alpha
            assert abs(ya - y1) <= 1e-15 * max(abs(ya), 1e-300) + 1e-300, (alpha, x)
            ga = o.grad_f64(x, 1.0, alpha)[0]
            g1 = o.grad_f64(alpha * x, 1.0, 1.0)[0]
            assert abs(ga - g1) <= 1e-14 * (1 + abs(alpha * x)), (alpha, x, ga, g1)


def pin_asymptotes(o):
    assert abs(o.swish_f64(40.0, 1.0) / 40.0 - 1.0) <= 1e-15
    assert abs(o.swish_f64(-40.0, 1.0)) < 1e-15
    assert o.swish_f64(-40.0, 1.0) < 0.0
    assert abs(o.grad_f64(40.0, 1.0, 1.0)[0] - 1.0) < 1e-14
    assert abs(o.grad_f64(-40.0, 1.0, 1.0)[0]) < 1e-14
    # Far out, sigma rounds to exactly 1 and 0 in binary64.
    assert o.swish_f64(1e6, 1.0) == 1e6
    assert o.swish_f64(-1e6, 1.0) == 0.0


def pin_stationary_point(o):
    """y'(x*) = 0 at x* = -(1 + W(1/e)) / alpha, where y(x*) = -W(1/e) / alpha."""
    from scipy.special import lambertw
    w = float(lambertw(math.exp(-1.0)).real)
    for alpha in ALPHAS:
        xs = -(1.0 + w) / alpha
        g, m = o.grad_f64(xs, 1.0, alpha)
        assert abs(g) <= 1e-15 * m, (alpha, g)
        y = o.swish_f64(xs, alpha)
        assert abs(y - (-w / alpha)) <= 1e-15 * abs(w / alpha), (alpha, y)


def pin_finite_differences(o):
    """Central differences of the oracle's own forward match its backward."""
    for alpha in ALPHAS:
        for x in _grid(-20.0, 20.0, 500, 13):
            h = 1e-5 * max(1.0, abs(x))
            fd = (o.swish_f64(x + h, alpha) - o.swish_f64(x - h, alpha)) / (2 * h)
            g, m = o.grad_f64(x, 1.0, alpha)
            assert abs(fd - g) <= 1e-8 * max(m, 1e-3), (alpha, x, fd, g)
    # dy enters linearly.
    for dy in (-3.0, 0.25, 7.5):
        for x in (-2.0, 0.3, 5.0):
            g1 = o.grad_f64(x, 1.0, 1.5)[0]
            gd = o.grad_f64(x, dy, 1.5)[0]
            assert abs(gd - dy * g1) <= 1e-15 * abs(dy * g1) + 1e-300


def pin_torch_autograd_naive(o):
    """The pages' claim that the saved-input backward equals autograd of the
    plain module: binary64 PyTorch CPU autograd of input * sigmoid(alpha input)."""
    import torch
    rng = np.random.default_rng(17)
    x = np.concatenate([rng.uniform(-30, 30, 600), rng.standard_normal(600) * 3])
    dy = rng.standard_normal(x.size)
    for alpha in ALPHAS:
        xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
        y = xt * torch.sigmoid(alpha * xt)
        y.backward(torch.tensor(dy, dtype=torch.float64))
        gt = xt.grad.numpy()
        y = y.detach().numpy()
        for i in range(x.size):
            g, m = o.grad_f64(x[i], dy[i], alpha)
            assert abs(g - gt[i]) <= 1e-14 * max(m, 1e-300), (alpha, x[i], g, gt[i])
            yo = o.swish_f64(x[i], alpha)
            assert abs(yo - float(y[i])) <= 4e-15 * max(abs(yo), 1e-300), (alpha, x[i])


def pin_error_scale(o):
    """m = |dy| s (1 + |t| (1-s)) bounds |g|, equals it for t >= 0 and stays
    within a factor 2 of it for t <= -4."""
    for alpha in ALPHAS:
        for x in _grid(-40.0, 40.0, 400, 19):
            g, m = o.grad_f64(x, -2.0, alpha)
            assert m >= abs(g) * (1 - 1e-15), (alpha, x, g, m)
            t = alpha * x
            if t >= 0:
                assert abs(m - abs(g)) <= 1e-15 * m, (alpha, x)
            elif t <= -4 and abs(g) > 0:
                assert m <= 2.0 * abs(g), (alpha, x, g, m)


def pin_nan_propagation(o):
    assert math.isnan(o.swish_f64(float("nan"), 1.0))
    assert math.isnan(o.grad_f64(float("nan"), 1.0, 1.0)[0])
    assert math.isnan(o.grad_f64(1.0, float("nan"), 1.0)[0])
    x = np.array([np.nan, 1.0, -2.0], dtype=np.float32)
    y = o.fwd(x, 1.0)
    assert np.isnan(y[0]) and not np.isnan(y[1:]).any()
    dx, _ = o.bwd(x, np.array([1.0, np.nan, 1.0], dtype=np.float32), 1.0)
    assert np.isnan(dx[0]) and np.isnan(dx[1]) and not np.isnan(dx[2])


# --------------------------------------------------------------------------
# Rounding.
# --------------------------------------------------------------------------

def _rounding_probe_values():
    rng = np.random.default_rng(23)
    e = rng.uniform(-160, 130, 4000)
    mant = rng.uniform(1.0, 2.0, 4000)
    v = np.ldexp(mant, e.astype(int)) * np.where(rng.random(4000) < 0.5, -1, 1)
    return np.concatenate([v, [0.0, -0.0, 1.0, -1.0, 2.0 ** -149, 2.0 ** -150,
                               3 * 2.0 ** -151, 2.0 ** -126, 3.4028235677973366e38,
                               3.4028235677973366e38 * (1 + 2.0 ** -25), 1e39]])


def pin_round_f32(o):
    for v in _rounding_probe_values():
        with np.errstate(over="ignore"):
            want = np.float64(v).astype(np.float32)
        got = o.round_f32(float(v))
        assert got.tobytes() == want.tobytes(), (v, got, want)


def _bf16_exact_nearest(v: float) -> int:
    """Nearest bfloat16 to v (ties to even), by exact rational arithmetic."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    sign = 0x8000 if v < 0 else 0
    a = Fraction(abs(v))
    # bfloat16 magnitudes: subnormal j * 2^-133 (j < 128); normal
    # (128 + f) * 2^(E-134) for E = 1..254.  Enumerate the exponent.
    if a < Fraction(2) ** -126:
        q = Fraction(2) ** -133
        E = 0
    else:
        E = 1
        while E < 254 and a >= Fraction(2) ** (E - 126):
            E += 1
        q = Fraction(2) ** (E - 134)
    k = a / q
    lo = math.floor(k)
    rem = k - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    # lo counts spacings above the start of the binade (or from zero).
    if E == 0:
        bits = lo  # subnormal field; 128 carries into the first normal binade
    else:
        bits = (E << 7) + (lo - 128)
    if bits >= 0x7F80:
        bits = 0x7F80
    return sign | bits


def pin_round_bf16_exact(o):
    rng = np.random.default_rng(29)
    vals = list(_rounding_probe_values()[:1500])
    # Values a hair off the halfway points, where rounding through binary32
    # first would give the wrong answer.
    for _ in range(300):
        b = int(rng.integers(0x0001, 0x7F7F))
        lo = (np.uint32(b) << 16).view(np.float32)
        hi = (np.uint32(b + 1) << 16).view(np.float32)
        mid = (float(lo) + float(hi)) / 2
        vals += [mid, mid * (1 + 2.0 ** -40), mid * (1 - 2.0 ** -40), -mid]
    for v in vals:
        assert o.round_bf16(float(v)) == _bf16_exact_nearest(float(v)), v


def pin_round_bf16_vs_torch(o):
    """binary32-representable values: torch's float32 -> bfloat16 cast (RNE)."""
    import torch
    allb = np.arange(1 << 16, dtype=np.uint32)
    f = (allb << 16).view(np.float32)
    nxt = ((allb + 1) << 16).view(np.float32)
    cand = [f, (f.astype(np.float64) + nxt.astype(np.float64)) / 2]
    with np.errstate(invalid="ignore", over="ignore"):
        v = np.concatenate(cand).astype(np.float32)
    v = v[np.isfinite(v)][::7]
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    for i in range(v.size):
        assert o.round_bf16(float(v[i])) == int(want[i]), (v[i], want[i])


# --------------------------------------------------------------------------
# Array drivers.
# --------------------------------------------------------------------------

def pin_array_drivers(o):
    """Array drivers = scalar binary64 value rounded, for both encodings and
    for any thread split."""
    rng = np.random.default_rng(31)
    x64 = np.concatenate([rng.standard_normal(3000) * 5, rng.uniform(-120, 120, 1000),
                          [0.0, -0.0, 1e-40, -1e-40, 3e38, -3e38]])
    dy64 = rng.standard_normal(x64.size)
    x32 = x64.astype(np.float32)
    dy32 = dy64.astype(np.float32)
    u = x32.view(np.uint32)
    xb = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    ub = dy32.view(np.uint32)
    dyb = ((ub + 0x7FFF + ((ub >> 16) & 1)) >> 16).astype(np.uint16)
    for alpha in (1.0, 1.5):
        y1 = o.fwd(x32, alpha, threads=1)
        y7 = o.fwd(x32, alpha, threads=7)
        assert y1.tobytes() == y7.tobytes()
        d1, m1 = o.bwd(x32, dy32, alpha, threads=1)
        d5, m5 = o.bwd(x32, dy32, alpha, threads=5)
        assert d1.tobytes() == d5.tobytes() and np.array_equal(m1, m5)
        yb = o.fwd(xb, alpha, threads=3)
        db, _ = o.bwd(xb, dyb, alpha, threads=3)
        xbf = (xb.astype(np.uint32) << 16).view(np.float32)
        dybf = (dyb.astype(np.uint32) << 16).view(np.float32)
        for i in range(x32.size):
            a = float(np.float32(alpha))
            assert y1[i].tobytes() == o.round_f32(o.swish_f64(float(x32[i]), a)).tobytes()
            g, m = o.grad_f64(float(x32[i]), float(dy32[i]), a)
            assert d1[i].tobytes() == o.round_f32(g).tobytes()
            assert m1[i] == m
            assert int(yb[i]) == o.round_bf16(o.swish_f64(float(xbf[i]), a))
            assert int(db[i]) == o.round_bf16(o.grad_f64(float(xbf[i]), float(dybf[i]), a)[0])


def pin_bf16_exhaustive_forward(o):
    """Every finite bfloat16 input at alpha 1: the array driver agrees with
    the mpmath-free closed form x / (1 + exp(-x)) evaluated in binary64 by
    numpy, rounded exactly by Fraction where the two neighbours are close."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]
    xf = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        ref = xf / (1.0 + np.exp(-xf))
    got = o.fwd(b, 1.0, threads=4)
    mism = np.nonzero(got != np.array([o.round_bf16(v) for v in ref], dtype=np.uint16))[0]
    assert mism.size == 0, mism[:10]
    # And the rounding of those references agrees with exact rational rounding.
    for i in range(0, b.size, 97):
        assert int(got[i]) == _bf16_exact_nearest(float(ref[i])), i


# --------------------------------------------------------------------------
# Page-3 byte accounting.
# --------------------------------------------------------------------------

def pin_page3_sizing(_o=None):
    from memory_efficient_activation_amd import accounting as acc
    from memory_efficient_activation_amd import inputs
    g = _golden("page3_sizing.json")
    n = acc.activation_elements(g["given"]["B"], g["given"]["T"], g["given"]["d"])
    assert n == g["elements"]
    assert round(n / 1e7, 2) == g["elements_rounded"] / 1e7
    assert int(np.prod(inputs.CONFIG_SHAPES[3][0])) == n
    assert int(np.prod(inputs.CONFIG_SHAPES[4][0])) == n
    b16 = acc.tensor_bytes(n, "bf16")
    b32 = acc.tensor_bytes(n, "f32")
    assert round(b16 / 1e6, 1) == g["mb_bf16"]
    assert round(b32 / 1e6, 1) == g["mb_fp32"]
    assert round(b16 / 1e5) * 1e5 == g["bytes_bf16_rounded"]
    assert 2 * b16 == b32  # Check: bf16 is exactly half of fp32
    L = g["given"]["L"]
    assert round(acc.stored_across_layers(n, "bf16", L) / 1e9, 2) == g["gb_bf16_all_layers"]
    assert round(acc.stored_across_layers(n, "f32", L) / 1e9, 2) == g["gb_fp32_all_layers"]
    assert acc.retained_bytes(n, "bf16") == b16
    assert acc.retained_bytes(n, "bf16", naive=True) == 3 * b16
    assert acc.fwd_bytes(n, "bf16") + acc.bwd_bytes(n, "bf16") == 671_088_640




# --------------------------------------------------------------------------
# The activation family of "What activations cost, in memory and in
# arithmetic" (Given).
# --------------------------------------------------------------------------

FAMILY = ("relu", "leaky_relu", "sigmoid", "tanh", "gelu_erf", "gelu_tanh")
LEAKY_SLOPE = 0.01


def _param(act):
    return LEAKY_SLOPE if act == "leaky_relu" else 0.0


def pin_family_special_values(o):
    for c in _golden("activation_family_special_values.json")["cases"]:
        assert o.act_f64(c["act"], c["x"], c["p"]) == c["value"], c
        assert o.act_grad_f64(c["act"], c["x"], 1.0, c["p"])[0] == c["grad"], c


def _mp_family(act, p):
    import mpmath
    a = mpmath.mpf(p)
    if act == "relu":
        return lambda u: u if u > 0 else mpmath.mpf(0)
    if act == "leaky_relu":
        return lambda u: u if u > 0 else a * u
    if act == "sigmoid":
        return lambda u: 1 / (1 + mpmath.exp(-u))
    if act == "tanh":
        return mpmath.tanh
    if act == "gelu_erf":
        return lambda u: u * mpmath.ncdf(u)
    k = mpmath.sqrt(2 / mpmath.pi)
    return lambda u: u * (1 + mpmath.tanh(k * (u + mpmath.mpf("0.044715") * u ** 3))) / 2


def pin_family_mpmath(o):
    """Each activation and its derivative at 60 digits (mpmath's own
    functions, the textbook formulas), including the far tails."""
    import mpmath
    mpmath.mp.dps = 60
    for act in FAMILY:
        p = _param(act)
        f = _mp_family(act, p)
        for x in np.concatenate([_grid(-30.0, 30.0, 40, 41), [-0.3, 0.7, 1e-3, -1e-3]]):
            # (1 + tanh u) / 2 cancels to about e^(2u): carry enough digits.
            mpmath.mp.dps = 60 + (int(0.04 * abs(x) ** 3) if act == "gelu_tanh" else 0)
            X = mpmath.mpf(float(x))
            ref = f(X)
            y = o.act_f64(act, x, p)
            # Where the function behaves like exp(-z), binary64 rounding of
            # the argument z costs about |z| ulps: the condition number.
            z = {"sigmoid": abs(x), "tanh": 2 * abs(x), "gelu_erf": x * x,
                 "gelu_tanh": 0.08 * abs(x) ** 3 + 2 * abs(x)}.get(act, 0.0)
            cond = 1.0 + z
            assert abs(y - float(ref)) <= 1e-14 * cond * abs(float(ref)) + 1e-300, (act, x, y, ref)
            if act in ("relu", "leaky_relu") and abs(x) < 1e-2:
                continue  # kink at 0: no two-sided derivative
            dref = mpmath.diff(f, X)
            g, m = o.act_grad_f64(act, x, 1.0, p)
            assert abs(g - float(dref)) <= 1e-13 * cond * max(m, 1e-300) + 1e-300, (act, x, g, dref)


def pin_family_torch_autograd(o):
    """Binary64 PyTorch CPU autograd of torch's own activations (an
    independent implementation), where torch itself does not cancel."""
    import torch
    import torch.nn.functional as F
    fns = {"relu": torch.relu, "leaky_relu": lambda t: F.leaky_relu(t, LEAKY_SLOPE),
           "sigmoid": torch.sigmoid, "tanh": torch.tanh,
           "gelu_erf": lambda t: F.gelu(t, approximate="none"),
           "gelu_tanh": lambda t: F.gelu(t, approximate="tanh")}
    rng = np.random.default_rng(43)
    x_all = np.concatenate([rng.uniform(-4, 30, 500), rng.standard_normal(500) * 2, [0.0, 1e-6, -1e-6]])
    dy_all = rng.standard_normal(x_all.size)
    # torch's own backward works from the output (1 - y, 1 - y^2, 1 + erf),
    # which cancels in the tails: compare where it keeps 13 digits.
    limit = {"sigmoid": 6.0, "tanh": 3.0, "gelu_erf": 3.0, "gelu_tanh": 3.0}
    for act, fn in fns.items():
        p = _param(act)
        lim = limit.get(act, np.inf)
        x = x_all[np.abs(x_all) <= lim]
        dy = dy_all[np.abs(x_all) <= lim]
        xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
        y = fn(xt)
        y.backward(torch.tensor(dy, dtype=torch.float64))
        gt, yt = xt.grad.numpy(), y.detach().numpy()
        for i in range(x.size):
            g, m = o.act_grad_f64(act, x[i], dy[i], p)
            assert abs(g - gt[i]) <= 1e-12 * max(m, 1e-300) + 1e-300, (act, x[i], g, gt[i])
            yo = o.act_f64(act, x[i], p)
            assert abs(yo - yt[i]) <= 1e-12 * abs(yo) + 1e-300, (act, x[i], yo, yt[i])


def pin_family_library_routines(o):
    from scipy.special import expit, ndtr
    for x in _grid(-40.0, 40.0, 300, 47):
        assert abs(o.act_f64("sigmoid", x) - expit(x)) <= 1e-15 * expit(x) + 1e-320
        assert abs(o.act_f64("tanh", x) - np.tanh(x)) <= 2e-16 * abs(np.tanh(x)) + 1e-320
        if x > -25.0:  # scipy's ndtr loses relative accuracy further out
            ge = x * ndtr(x)
            assert abs(o.act_f64("gelu_erf", x) - ge) <= 1e-13 * abs(ge) + 1e-320, x


def pin_family_identities(o):
    """sigma(x) + sigma(-x) = 1, tanh odd, GELU(x) - GELU(-x) = x for both
    variants (u is odd in x), ReLU(x) - ReLU(-x) = x; derivatives of the
    symmetric ones are even."""
    for x in _grid(-20.0, 20.0, 200, 53):
        assert abs(o.act_f64("sigmoid", x) + o.act_f64("sigmoid", -x) - 1) <= 4.5e-16
        assert o.act_f64("tanh", -x) == -o.act_f64("tanh", x)
        assert o.act_grad_f64("tanh", x, 1.0)[0] == o.act_grad_f64("tanh", -x, 1.0)[0]
        gs, gsm = o.act_grad_f64("sigmoid", x, 1.0)[0], o.act_grad_f64("sigmoid", -x, 1.0)[0]
        assert abs(gs - gsm) <= 1e-16 * gs
        for act in ("gelu_erf", "gelu_tanh"):
            d = o.act_f64(act, x) - o.act_f64(act, -x)
            assert abs(d - x) <= 1e-15 * max(abs(x), 1.0), (act, x, d)
            gsum = o.act_grad_f64(act, x, 1.0)[0] + o.act_grad_f64(act, -x, 1.0)[0]
            assert abs(gsum - 1.0) <= 1e-13 * (1 + x * x), (act, x, gsum)
        assert o.act_f64("relu", x) - o.act_f64("relu", -x) == x


def pin_family_finite_differences(o):
    for act in FAMILY:
        p = _param(act)
        for x in _grid(-12.0, 12.0, 300, 59):
            if act in ("relu", "leaky_relu") and abs(x) < 1e-3:
                continue
            h = 1e-5 * max(1.0, abs(x))
            fd = (o.act_f64(act, x + h, p) - o.act_f64(act, x - h, p)) / (2 * h)
            g, m = o.act_grad_f64(act, x, 1.0, p)
            assert abs(fd - g) <= 1e-8 * max(m, 1e-3), (act, x, fd, g)


def pin_family_array_drivers(o):
    rng = np.random.default_rng(61)
    x64 = np.concatenate([rng.standard_normal(1500) * 5, rng.uniform(-100, 100, 500),
                          [0.0, -0.0, 1e-40, -1e-40, 3e38, -3e38]])
    dy64 = rng.standard_normal(x64.size)
    x32, dy32 = x64.astype(np.float32), dy64.astype(np.float32)
    u, ub = x32.view(np.uint32), dy32.view(np.uint32)
    xb = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    dyb = ((ub + 0x7FFF + ((ub >> 16) & 1)) >> 16).astype(np.uint16)
    xbf = (xb.astype(np.uint32) << 16).view(np.float32)
    dybf = (dyb.astype(np.uint32) << 16).view(np.float32)
    for act in FAMILY:
        p = float(np.float32(_param(act)))
        y1 = o.act_fwd(act, x32, p, threads=1)
        y5 = o.act_fwd(act, x32, p, threads=5)
        assert y1.tobytes() == y5.tobytes()
        d1, m1 = o.act_bwd(act, x32, dy32, p, threads=3)
        yb = o.act_fwd(act, xb, p, threads=2)
        db, _ = o.act_bwd(act, xb, dyb, p, threads=2)
        for i in range(x32.size):
            assert y1[i].tobytes() == o.round_f32(o.act_f64(act, float(x32[i]), p)).tobytes()
            g, m = o.act_grad_f64(act, float(x32[i]), float(dy32[i]), p)
            assert d1[i].tobytes() == o.round_f32(g).tobytes() and m1[i] == m
            assert int(yb[i]) == o.round_bf16(o.act_f64(act, float(xbf[i]), p))
            assert int(db[i]) == o.round_bf16(o.act_grad_f64(act, float(xbf[i]), float(dybf[i]), p)[0])
    # NaN in, NaN out.
    for act in FAMILY:
        assert math.isnan(o.act_f64(act, float("nan"), 0.01))
        assert math.isnan(o.act_grad_f64(act, float("nan"), 1.0, 0.01)[0])
        assert math.isnan(o.act_grad_f64(act, 1.0, float("nan"), 0.01)[0])



def pin_infinite_inputs(o):
    """x = +-inf gives the limits as x -> +-inf (parameter fixed), written
    as closed forms: Swish and both GELUs tend to x at +inf and to a zero of
    the sign of x at -inf, their derivatives to 1 and to -0; ReLU's value
    and slope tend to 0 at -inf, LeakyReLU's to -inf and its slope; sigmoid
    and tanh tend to their asymptotes with vanishing slope.  A zero
    parameter keeps IEEE 0 * inf = NaN.  The limits also agree with the
    oracle far out on the finite axis."""
    inf = float("inf")

    def same(a, b):
        return (math.isnan(a) and math.isnan(b)) or (a == b and math.copysign(1, a) == math.copysign(1, b))

    dy = -2.5
    want = {
        # act: (param, f(+inf), f(-inf), dy f'(+inf), dy f'(-inf))
        "swish": (1.0, inf, -0.0, dy, dy * -0.0),
        "relu": (0.0, inf, 0.0, dy, dy * 0.0),
        "leaky_relu": (0.01, inf, -inf, dy, dy * 0.01),
        "sigmoid": (0.0, 1.0, 0.0, dy * 0.0, dy * 0.0),
        "tanh": (0.0, 1.0, -1.0, dy * 0.0, dy * 0.0),
        "gelu_erf": (0.0, inf, -0.0, dy, dy * -0.0),
        "gelu_tanh": (0.0, inf, -0.0, dy, dy * -0.0),
    }
    for act, (p, fp, fm, gp, gm) in want.items():
        assert same(o.act_f64(act, inf, p), fp), act
        assert same(o.act_f64(act, -inf, p), fm), act
        assert same(o.act_grad_f64(act, inf, dy, p)[0], gp), act
        assert same(o.act_grad_f64(act, -inf, dy, p)[0], gm), act
        # Far out on the finite axis the values already sit at the limits.
        for x, lim in ((1e4, fp), (-1e4, fm)):
            v = o.act_f64(act, x, p)
            if math.isinf(lim):  # grows without bound, with the limit's sign
                assert math.copysign(1, v) == math.copysign(1, lim) and abs(v) >= 1e-2 * abs(x), (act, x, v)
            else:
                assert abs(v - lim) < 1e-12, (act, x, v)
    # Swish with a negative slope mirrors the limits; a zero slope is NaN.
    assert same(o.swish_f64(inf, -1.0), 0.0) and same(o.swish_f64(-inf, -1.0), -inf)
    assert same(o.grad_f64(inf, 1.0, -1.0)[0], -0.0) and same(o.grad_f64(-inf, 1.0, -1.0)[0], 1.0)
    assert math.isnan(o.swish_f64(inf, 0.0)) and math.isnan(o.grad_f64(-inf, 1.0, 0.0)[0])
    assert math.isnan(o.act_f64("leaky_relu", -inf, 0.0))
    # The array drivers round the limits like any other value.
    x = np.array([inf, -inf], dtype=np.float32)
    y = o.act_fwd("gelu_erf", x, 0.0)
    assert y[0] == inf and y[1] == 0.0 and math.copysign(1, y[1]) < 0


def pin_family_error_scale(o):
    """The error scale m of each backward is tight, not just an upper bound:
    it is the sum of the absolute values of the terms of dy f'(x), so it
    equals |dy f'(x)| wherever those terms share a sign -- every x for ReLU,
    LeakyReLU, sigmoid and tanh (one term each), x >= 0 for both GELUs -- and
    it bounds |dy f'(x)|, staying within 1.3 times it, where the GELU terms
    Phi and x phi differ in sign but x phi dominates (x <= -3: the ratio is
    (|x| + 1/|x|) / (|x| - 1/|x|) at leading order for erf, and likewise
    for the tanh form).  An inflated or loosened scale fails here."""
    for act in FAMILY:
        p = _param(act)
        for x in _grid(-30.0, 30.0, 300, 67):
            for dy in (1.0, -0.37):
                g, m = o.act_grad_f64(act, x, dy, p)
                assert m >= abs(g) * (1 - 1e-15), (act, x, g, m)
                if act in ("gelu_erf", "gelu_tanh"):
                    if x >= 0:
                        assert abs(m - abs(g)) <= 1e-15 * m, (act, x, g, m)
                    elif x <= -3.0 and g != 0.0:
                        assert m <= 1.3 * abs(g), (act, x, g, m)
                else:
                    assert m == abs(g), (act, x, g, m)
    # A case where the two GELU terms cancel exactly is where m is needed:
    # near the zero of GELU' (x = -0.7518 for erf) m stays of order Phi.
    g, m = o.act_grad_f64("gelu_erf", -0.7517915241, 1.0)
    assert abs(g) < 1e-9 and 0.4 < m < 0.5, (g, m)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
