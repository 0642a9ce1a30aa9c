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


# Tiles per launch of the vector kernel (the library's kMaxLaunchTiles).
LAUNCH_TILES = 1 << 30


def covered(p, n, esize, launch_tiles=None):
    """Element indices the kernels touch, by the kernels' own arithmetic:
    launch c of the vector path covers tiles [c L, (c + 1) L) of the body
    (L = LAUNCH_TILES) from a pointer at the start of its part; block b takes
    tiles b, b + grid, ... of its launch; the first launch also does the
    head and the last the tail."""
    E, TV = p.elems_per_vector, p.vectors_per_tile
    L = launch_tiles or LAUNCH_TILES
    seen = np.zeros(n, dtype=np.int32)
    if p.path == _lib.PATH_VECTOR:
        done = 0
        for c in range(p.launches):
            nt = min(p.tiles - c * L, L)
            vecs = min(nt * TV, p.nvec - c * L * TV)
            last_vecs = vecs - (nt - 1) * TV if nt else 0
            head = p.head if c == 0 else 0
            tail = p.tail if c + 1 == p.launches else 0
            base = 0 if c == 0 else p.head + done   # element offset of the launch's pointer
            for b in range(p.grid):
                t = b
                while t < nt:
                    nv = TV if t + 1 < nt else last_vecs
                    for thread in range(p.block):
                        for u in range(TV // p.block):
                            v = thread + u * p.block
                            if v < nv:
                                e0 = base + head + (t * TV + v) * E
                                seen[e0:e0 + E] += 1
                    t += p.grid
            for thread in range(head + tail):
                i = thread if thread < head else head + vecs * E + (thread - head)
                seen[base + i] += 1
            done += vecs * E
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
            assert p.launches == 1
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


@pytest.mark.parametrize("bwd", [0, 1])
def test_plan_grid_stays_below_the_thread_limit(lib, bwd):
    """grid x block must stay below 2^32 threads (the launch limit) for any
    n the header accepts: bfloat16 of 2^32 elements on the element path,
    2^35 + 2^20 on the vector path, and past 2^30 tiles (several launches)."""
    es = 2
    span = 1 << 46   # fake buffers far apart: no overlap for these sizes
    x, dy, out = BASE, BASE + span, BASE + 2 * span
    cases = [(x + 2, dy + 2 if bwd else None, out, 1 << 32, _lib.PATH_ELEMENT),
             (x, dy if bwd else None, out, (1 << 35) + (1 << 20), _lib.PATH_VECTOR),
             (x, dy if bwd else None, out, 1 << 42, _lib.PATH_VECTOR)]
    for xp, dp, op, n, path in cases:
        st, p = plan(lib, xp, dp, op, n, _lib.BF16, bwd)
        assert st == _lib.OK and p.path == path, (n, st, p.path)
        assert p.grid * p.block < (1 << 32), (n, p.grid, p.block)
        if path == _lib.PATH_VECTOR:
            assert p.head + p.nvec * p.elems_per_vector + p.tail == n
            assert p.launches == -(-p.tiles // LAUNCH_TILES)
            assert p.grid <= min(p.tiles, LAUNCH_TILES)
    # Past 2^30 tiles: 2^42 bfloat16 elements are 2^39 vectors.
    p = plan(lib, x, dy if bwd else None, out, 1 << 42, _lib.BF16, bwd)[1]
    assert p.launches == (1 << 39) // p.vectors_per_tile // LAUNCH_TILES >= 2


def test_split_into_several_launches():
    """The test build with 3 tiles per launch (built by __graft_entry__.build())
    splits moderate tensors into several launches; the kernels' arithmetic,
    launch by launch, covers every element exactly once, with the head in
    the first launch and the tail in the last."""
    from memory_efficient_activation_amd import build as lib_build
    if not __import__("os").path.exists(lib_build.SPLIT_TEST_LIBRARY):
        pytest.fail("the split test build is missing (run __graft_entry__.build())")
    lib3 = _lib.library(lib_build.SPLIT_TEST_LIBRARY, lib_build.SPLIT_TEST_NAMES)
    L = lib_build.SPLIT_TEST_TILES
    rng = np.random.default_rng(5)
    for dtype, esize in ((_lib.F32, 4), (_lib.BF16, 2)):
        for bwd in (0, 1):
            for n in (1, 100, 511, 2048, 2049, 5000, 9 * 512 + 7, 40000):
                off = int(rng.integers(0, 16 // esize)) * esize
                x, dy, out = BASE + off, BASE + (1 << 30) + off, BASE + (2 << 30) + off
                st, p = plan(lib3, x, dy if bwd else None, out, n, dtype, bwd)
                assert st == _lib.OK and p.path == _lib.PATH_VECTOR
                assert p.launches == max(1, -(-p.tiles // L)), (n, p.tiles, p.launches)
                assert p.grid <= L
                seen = covered(p, n, esize, launch_tiles=L)
                assert (seen == 1).all(), (dtype, bwd, n, off)
