"""The product path has no CPU fallback: every public call refuses CPU
tensors, a missing library is an error, and no module of the package uses
the oracle (which only the tests, smoke() and the bench's CPU baseline
run)."""

import ast
import os

import pytest
import torch

import memory_efficient_activation_amd as mea
from memory_efficient_activation_amd import _lib, dense, fft

PKG = os.path.dirname(os.path.abspath(mea.__file__))


def _refuses(fn, *args):
    with pytest.raises(RuntimeError, match="no CPU path"):
        fn(*args)


def test_cpu_tensors_are_refused():
    x = torch.randn(64)
    _refuses(mea.swish_fwd, x)
    _refuses(mea.swish_bwd, x, x)
    _refuses(mea.swish_fwd_grouped, [x, x])
    _refuses(mea.swish_bwd_grouped, [x], [x])
    _refuses(mea.act_fwd, "gelu", x)
    _refuses(mea.act_bwd, "gelu", x, x)
    _refuses(mea.MemoryEfficientSwish(1.0), x)
    _refuses(mea.MemoryEfficientActivation("relu"), x)
    _refuses(dense.bn_stats, torch.randn(2, 3, 4))
    _refuses(fft.r2c, torch.randn(4, 8, 8), 8)
    _refuses(fft.fprop, torch.randn(2, 3, 8, 8), torch.randn(4, 3, 3, 3))


def test_missing_library_is_an_error(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIBRARY", str(tmp_path / "libmeswish.so"))
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.library()


def test_package_never_imports_the_oracle():
    for name in sorted(os.listdir(PKG)):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(PKG, name)).read())
        for node in ast.walk(tree):
            mods = []
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            for m in mods:
                assert not m.split(".")[0] == "oracle", (name, m)
