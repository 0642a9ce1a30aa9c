"""The README's usage example runs as written (on the GPU)."""

import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs():
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert len(blocks) == 1
    env = {}
    exec(compile(blocks[0], "README.md", "exec"), env)
    torch.cuda.synchronize()
    assert env["x"].grad is not None and env["x"].grad.shape == env["x"].shape
    assert [t.shape for t in env["ys"]] == [(1000,), (4096,), (77,)]
    assert env["y"].shape == (128, 256, 26, 26)
