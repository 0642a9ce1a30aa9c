"""The synthetic DenseNet-BC experiment on the GPU (README of
efficient_densenet_pytorch, "A memory-efficient implementation of
DenseNets", Motivation and Performance): the shared-buffer network keeps
far fewer bytes between forward and backward than the plain one, and its
loss and gradients are at least as close to a binary64 evaluation."""

import pytest

from memory_efficient_activation_amd import dense_experiment as dx

from gpu_util import say

pytestmark = pytest.mark.gpu


def test_densenet_bc40_shared_buffers_save_the_quadratic_maps():
    r = dx.measure(depth=40, batch=16, reps=1)
    say(f"[dense-model] {r}")
    nv, ef = r["naive"], r["memory_efficient"]
    assert r["rel_loss_diff"] < 1e-5
    saved = nv["retained_after_forward_bytes"] - ef["retained_after_forward_bytes"]
    # The plain network keeps each layer's concatenation and its normalized
    # form; the efficient one keeps each layer's own output instead (and
    # one shared buffer).
    assert saved > 0.5 * r["concat_and_bn_maps_bytes"]
    assert ef["peak_step_bytes"] < nv["peak_step_bytes"]


def test_densenet_bc40_gradients_against_binary64():
    """Both GPU networks against the plain network in binary64 on the CPU.
    The binary32 plain network drifts by up to a few percent on some
    gradients (with or without MIOpen); the efficient network must never
    be further off than it, parameter by parameter."""
    r = dx.errors_vs_binary64(depth=40, batch=16)
    nv, ef = r["naive"], r["memory_efficient"]
    worst_n = max(nv["grad_rel_err"].items(), key=lambda kv: kv[1])
    worst_e = max(ef["grad_rel_err"].items(), key=lambda kv: kv[1])
    say(f"[dense-model] vs binary64: loss err naive {nv['loss_rel_err']:.2e} efficient "
        f"{ef['loss_rel_err']:.2e}; worst grad err naive {worst_n}, efficient {worst_e}")
    assert ef["loss_rel_err"] < 1e-6
    for k, e in ef["grad_rel_err"].items():
        assert e <= 1.5 * nv["grad_rel_err"][k] + 1e-4, (k, e, nv["grad_rel_err"][k])


def test_densenet_bc40_step_under_graph_capture():
    """The training step of both networks captured into a HIP graph: every
    checked replay (eager work between replays) gives the eager step's loss
    and gradients."""
    r = dx.measure_graph(depth=40, batch=16, reps=5, checks=3)
    say(f"[dense-model] graph-captured step: {r}")
    for name in ("naive", "memory_efficient"):
        assert r[name]["replay_vs_eager_loss_rel"] <= 1e-6, (name, r[name])
        assert r[name]["replay_vs_eager_grad_rel"] <= 1e-4, (name, r[name])
