"""The module-level memory experiment on the GPU (blog post "Memory
efficient Swish", "How much GPU memory is saved?" and "Why simple Swish
implementation is inefficient?"): the memory-efficient network keeps exactly
one feature map less per activation than the plain one, and computes the
same loss and gradients."""

import pytest
import torch

from memory_efficient_activation_amd import memory_experiment as mx

from gpu_util import say

pytestmark = pytest.mark.gpu


def test_efficientnet_shapes_fp32_saves_one_map_per_activation():
    r = mx.measure("efficientnet", torch.float32, reps=1)
    say(f"[memory] efficientnet fp32: {r}")
    assert r["retained_saved_bytes"] == r["one_map_per_activation_bytes"]
    assert r["rel_loss_diff"] < 1e-5
    assert r["max_rel_grad_diff"] < 1e-4
    assert r["retained_saved_fraction"] > 0.3


def test_efficientnet_shapes_bf16():
    r = mx.measure("efficientnet", torch.bfloat16, reps=1)
    say(f"[memory] efficientnet bf16: {r}")
    assert r["retained_saved_bytes"] == r["one_map_per_activation_bytes"]
    assert r["peak_saved_fraction"] > 0.25
    # One rounding per element (fused, binary32 math) is at least as close
    # to the binary32 network as the eager bfloat16 ops are.
    ef, nv = r["memory_efficient"], r["naive"]
    assert ef["grad_rel_err_vs_f32"] <= nv["grad_rel_err_vs_f32"] * 1.05
    assert ef["loss_rel_err_vs_f32"] < 1e-2
