"""Host logic of libmeswish without a GPU: argument checks and the launch
plan (how a tensor is split into a scalar head, 16-byte vectors and a tail,
how many tiles and blocks), through ``meswish_plan``, which runs the same
code as swish_fwd / swish_bwd but launches nothing.

A small Python model of the vector kernel's index arithmetic then checks
that the plan covers every element exactly once and never leaves [0, n).
"""

import ctypes

import numpy as np
import pytest

from memory_efficient_activation_amd import _lib

BASE = 0x7F0000000000  # fake, 4 KiB-aligned device address: never dereferenced


@pytest.fixture(scope="module")
def lib():
    return _lib.library()


def plan(lib, x, dy, out, n, dtype, bwd, alpha=1.0):
    p = _lib.Plan()
    st = lib.meswish_plan(x, dy, out, n, alpha, dtype, bwd, ctypes.byref(p))
    return st, p


def covered(p, n, esize):
    """Element indices the vector kernel touches, by the kernel's arithmetic."""
    E, TV = p.elems_per_vector, p.vectors_per_tile
    seen = np.zeros(n, dtype=np.int32)
    if p.path == _lib.PATH_VECTOR:
        for b in range(p.grid):
            t0 = b * TV
            while t0 < p.nvec:
                for thread in range(p.block):
                    for u in range(TV // p.block):
                        v = t0 + thread + u * p.block
                        if v < p.nvec:
                            seen[p.head + v * E: p.head + (v + 1) * E] += 1
                t0 += p.grid * TV
        for thread in range(p.head + p.tail):
            i = thread if thread < p.head else p.head + p.nvec * E + (thread - p.head)
            seen[i] += 1
    else:
        for b in range(p.grid):
            i = b * p.block
            while i < n:
                for thread in range(p.block):
                    if i + thread < n:
                        seen[i + thread] += 1
                i += p.grid * p.block
    return seen


@pytest.mark.parametrize("dtype,esize", [(_lib.F32, 4), (_lib.BF16, 2)])
@pytest.mark.parametrize("bwd", [0, 1])
def test_plan_splits_and_covers(lib, dtype, esize, bwd):
    rng = np.random.default_rng(7 + dtype + 2 * bwd)
    sizes = list(range(0, 40)) + [255, 256, 257, 2047, 2048, 2049, 4096 * 3 + 5]
    for n in sizes:
        for _ in range(4):
            ox, od, oo = (int(v) * esize for v in rng.integers(0, 16 // esize, 3))
            if rng.random() < 0.5:
                od = oo = ox  # congruent pointers: vector path
            x = BASE + ox
            dy = BASE + (1 << 30) + od
            out = BASE + (2 << 30) + oo
            st, p = plan(lib, x, dy if bwd else None, out, n, dtype, bwd)
            assert st == _lib.OK
            if n == 0:
                assert p.path == _lib.PATH_NONE
                continue
            congruent = (ox % 16 == oo % 16) and (not bwd or od % 16 == ox % 16)
            assert p.elems_per_vector == 16 // esize
            assert p.block in (64, 256) and p.vectors_per_tile % p.block == 0
            if congruent:
                assert p.path == _lib.PATH_VECTOR
                assert p.head + p.nvec * p.elems_per_vector + p.tail == n
                assert 0 <= p.head < 16 // esize and 0 <= p.tail
                assert p.head == n or (x + p.head * esize) % 16 == 0
                assert p.tail < p.elems_per_vector or p.nvec == 0
                assert p.tiles == -(-p.nvec // p.vectors_per_tile)
            else:
                assert p.path == _lib.PATH_ELEMENT and p.tail == n
                assert p.tiles == -(-n // p.vectors_per_tile)
            assert 1 <= p.grid <= max(p.tiles, 1)
            if n <= 4096 * 3 + 5:
                seen = covered(p, n, esize)
                assert (seen == 1).all(), (n, ox, od, oo, p.path)


def test_plan_rejections_match_the_calls(lib):
    """Every rejection of swish_fwd/swish_bwd, checked on fake addresses
    (safe: the plan launches nothing)."""
    x, y = BASE, BASE + (1 << 30)
    nan = float("nan")
    assert plan(lib, x, None, y, 16, 9, 0)[0] == _lib.EINVAL           # dtype
    assert plan(lib, x, None, y, 16, _lib.F32, 0, nan)[0] == _lib.EINVAL
    assert plan(lib, None, None, y, 16, _lib.F32, 0)[0] == _lib.EINVAL
    assert plan(lib, x, None, None, 16, _lib.F32, 0)[0] == _lib.EINVAL
    assert plan(lib, x, None, y, 16, _lib.F32, 1)[0] == _lib.EINVAL    # bwd needs dy
    assert plan(lib, x + 2, None, y, 16, _lib.F32, 0)[0] == _lib.EINVAL  # element misalignment
    assert plan(lib, x + 1, None, y, 16, _lib.BF16, 0)[0] == _lib.EINVAL
    assert plan(lib, x, None, y, 1 << 62, _lib.F32, 0)[0] == _lib.EINVAL  # n too large
    # Aliasing: exact is fine, partial is not.
    assert plan(lib, x, None, x, 1024, _lib.F32, 0)[0] == _lib.OK
    assert plan(lib, x, None, x + 64, 1024, _lib.F32, 0)[0] == _lib.EALIAS
    assert plan(lib, x + 64, None, x, 1024, _lib.F32, 0)[0] == _lib.EALIAS
    assert plan(lib, x, x + 4096, x + 4096, 1024, _lib.F32, 1)[0] == _lib.OK     # dx == dy
    assert plan(lib, x, x + 4096, x, 1024, _lib.F32, 1)[0] == _lib.OK            # dx == x
    assert plan(lib, x, x + 4096, x + 4100, 1024, _lib.F32, 1)[0] == _lib.EALIAS
    assert plan(lib, x, x + 2, y, 1024, _lib.BF16, 1)[0] == _lib.OK  # inputs may overlap
    # Adjacent, non-overlapping ranges are fine.
    assert plan(lib, x, None, x + 4096, 1024, _lib.F32, 0)[0] == _lib.OK
    st, p = plan(lib, x, None, y, 0, _lib.F32, 0)
    assert st == _lib.OK and p.path == _lib.PATH_NONE
    assert lib.meswish_plan(x, None, y, 16, 1.0, _lib.F32, 0, None) == _lib.EINVAL
