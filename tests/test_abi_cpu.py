"""The C-ABI library: it loads, it exports every symbol include/meswish.h
declares, and its host-side argument checks answer without a GPU.

No compute call is made here: every call below is rejected (or is a no-op)
before anything is launched.
"""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "meswish.h")
LIB = os.path.join(ROOT, "memory_efficient_activation_amd", "libmeswish.so")


def _header_text():
    with open(HEADER) as f:
        text = f.read()
    return re.sub(r"/\*.*?\*/", "", text, flags=re.S)


def declared_functions():
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", _header_text())))


def declared_enum(name):
    body = re.search(r"typedef enum\s*\{([^{}]*)\}\s*" + name + ";", _header_text()).group(1)
    return {k: int(v) for k, v in re.findall(r"(\w+)\s*=\s*(\d+)", body)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmeswish.so is not built (run __graft_entry__.build())")
    from memory_efficient_activation_amd import _lib
    return _lib.library()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "meswish_act_bwd", "meswish_act_fwd",
        "meswish_copy", "meswish_plan", "meswish_strerror", "meswish_version", "swish_bwd",
        "swish_bwd_grouped", "swish_fwd", "swish_fwd_grouped"])


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name), name


def test_binding_constants_match_header(lib):
    from memory_efficient_activation_amd import _lib
    st = declared_enum("meswish_status")
    assert st == {"MESWISH_OK": _lib.OK, "MESWISH_EINVAL": _lib.EINVAL,
                  "MESWISH_EALIAS": _lib.EALIAS, "MESWISH_EHIP": _lib.EHIP,
                  "MESWISH_ETOOMANY": _lib.ETOOMANY}
    assert declared_enum("meswish_dtype") == {"MESWISH_F32": _lib.F32, "MESWISH_BF16": _lib.BF16}
    acts = declared_enum("meswish_act")
    assert {k[len("MESWISH_ACT_"):].lower(): v for k, v in acts.items()} == {
        ("gelu_erf" if k == "gelu" else k): v for k, v in _lib.ACTS.items()}
    m = re.search(r"#define MESWISH_MAX_GROUP (\d+)", _header_text())
    assert int(m.group(1)) == _lib.MAX_GROUP
    assert set(_lib.EXPORTED) == set(declared_functions())
    m = re.findall(r"MESWISH_PATH_(\w+)\s*=\s*(-?\d+)", _header_text())
    assert {k: int(v) for k, v in m} == {"NONE": _lib.PATH_NONE, "VECTOR": _lib.PATH_VECTOR,
                                         "ELEMENT": _lib.PATH_ELEMENT}
    fields = re.search(r"typedef struct \{([^{}]*)\}\s*meswish_plan_t;", _header_text()).group(1)
    names = re.findall(r"(\w+);", fields)
    assert names == [f[0] for f in _lib.Plan._fields_]
    # Descriptor layouts: pointer, pointer, size_t (+ one more pointer for bwd).
    assert ctypes.sizeof(_lib.FwdDesc) == 24 and ctypes.sizeof(_lib.BwdDesc) == 32


def test_strerror_and_version(lib):
    for code in range(5):
        msg = lib.meswish_strerror(code)
        assert isinstance(msg, bytes) and msg
    assert lib.meswish_strerror(99) == b"unknown status"
    assert lib.meswish_version() >= 100


def test_rejections_before_launch(lib):
    from memory_efficient_activation_amd import _lib
    nan, inf = float("nan"), float("inf")
    # Unknown dtype, non-finite alpha: rejected before any pointer is looked at.
    assert lib.swish_fwd(None, None, 16, 1.0, 7, None) == _lib.EINVAL
    assert lib.swish_fwd(None, None, 16, nan, _lib.F32, None) == _lib.EINVAL
    assert lib.swish_bwd(None, None, None, 16, inf, _lib.BF16, None) == _lib.EINVAL
    # NULL pointers with n > 0.
    assert lib.swish_fwd(None, None, 16, 1.0, _lib.F32, None) == _lib.EINVAL
    assert lib.swish_bwd(None, None, None, 16, 1.0, _lib.F32, None) == _lib.EINVAL
    # n == 0 is a no-op, even with NULL pointers.
    assert lib.swish_fwd(None, None, 0, 1.0, _lib.F32, None) == _lib.OK
    assert lib.swish_bwd(None, None, None, 0, 1.0, _lib.BF16, None) == _lib.OK
    # Grouped: counts.
    assert lib.swish_fwd_grouped(None, -1, 1.0, _lib.F32, None) == _lib.EINVAL
    assert lib.swish_fwd_grouped(None, 3, 1.0, _lib.F32, None) == _lib.EINVAL
    assert lib.swish_fwd_grouped(None, 0, 1.0, _lib.F32, None) == _lib.OK
    d = (_lib.FwdDesc * 65)()
    assert lib.swish_fwd_grouped(d, 65, 1.0, _lib.F32, None) == _lib.ETOOMANY
    b = (_lib.BwdDesc * 65)()
    assert lib.swish_bwd_grouped(b, 65, 1.0, _lib.BF16, None) == _lib.ETOOMANY
    # Unknown activation; non-finite parameter.
    assert lib.meswish_act_fwd(7, None, None, 16, 1.0, _lib.F32, None) == _lib.EINVAL
    assert lib.meswish_act_bwd(-1, None, None, None, 16, 1.0, _lib.F32, None) == _lib.EINVAL
    assert lib.meswish_act_fwd(2, None, None, 16, nan, _lib.F32, None) == _lib.EINVAL
    assert lib.meswish_act_fwd(4, None, None, 0, 1.0, _lib.BF16, None) == _lib.OK
    # Copy helper: misaligned or odd sizes.
    assert lib.meswish_copy(None, None, 0, None) == _lib.OK
    assert lib.meswish_copy(None, None, 16, None) == _lib.EINVAL


def test_alias_and_alignment_rejections_without_gpu(lib):
    """Fake addresses are safe only where no GPU exists: a check that wrongly
    passed would try to launch.  The same cases run with real device buffers
    in the GPU suite."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("covered with real device buffers by the GPU tests")
    from memory_efficient_activation_amd import _lib
    base = 0x10000000
    # Partial overlap of y with x.
    assert lib.swish_fwd(base, base + 64, 1024, 1.0, _lib.F32, None) == _lib.EALIAS
    # dx overlapping dy partially.
    assert lib.swish_bwd(base, base + 8192, base + 8192 + 4, 1024, 1.0, _lib.F32, None) == _lib.EALIAS
    # Element misalignment.
    assert lib.swish_fwd(base + 1, base + 65536, 16, 1.0, _lib.BF16, None) == _lib.EINVAL
    assert lib.swish_fwd(base + 2, base + 65536, 16, 1.0, _lib.F32, None) == _lib.EINVAL
    # Grouped: output of tensor 0 coinciding with the input of tensor 1.
    d = (_lib.FwdDesc * 2)(_lib.FwdDesc(base, base + 4096, 256), _lib.FwdDesc(base + 4096, base + 8192, 256))
    assert lib.swish_fwd_grouped(d, 2, 1.0, _lib.F32, None) == _lib.EALIAS
