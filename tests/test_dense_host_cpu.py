"""Host-side arithmetic of the DenseNet-layer kernels, checked on the CPU.

The kernels split a vector index v of a channel into (row, position) by
the round-up multiply-shift division of Granlund and Montgomery, "Division
by invariant integers using multiplication" (1994): with s = ceil(log2 d)
and m = floor(2^32 (2^s - d) / d) + 1, v // d = (umulhi(v, m) + v) >> s in
32-bit arithmetic for every v < 2^31.  This checks that statement for the
divisors the layer shapes produce and for random ones, at the edges of
each quotient.
"""

import random


def magic(d):
    s = 0
    while (1 << s) < d:
        s += 1
    return (((1 << 32) * ((1 << s) - d)) // d + 1) & 0xFFFFFFFF, s


def fdiv(v, m, s):
    return ((((v * m) >> 32) + v) & 0xFFFFFFFF) >> s


def test_multiply_shift_division_is_exact_below_2_31():
    rng = random.Random(1)
    divisors = [1, 2, 3, 5, 7, 8, 16, 49, 64, 128, 196, 256, 585, 784, 1024, 3136, 12544,
                (1 << 30) + 1, (1 << 31) - 1] + [rng.randrange(1, 1 << 31) for _ in range(200)]
    for d in divisors:
        m, s = magic(d)
        vs = [0, 1, d - 1, d, d + 1, (1 << 31) - 1, (1 << 31) - 2]
        vs += [k * d + e for k in range(1, 40) for e in (-1, 0)]
        vs += [rng.randrange(0, 1 << 31) for _ in range(500)]
        for v in vs:
            if 0 <= v < (1 << 31):
                assert fdiv(v, m, s) == v // d, (d, v)
