"""Memory and time of a synthetic DenseNet-BC, plain vs shared-buffer.

The README of efficient_densenet_pytorch ("A memory-efficient implementation
of DenseNets") compares, in section Performance, the GPU memory and the time
per minibatch of a plain and an efficient DenseNet-BC with 100 layers at
batch size 64, and explains in section Motivation where the difference
comes from: the concatenation and batch-normalization outputs of every
layer, which the efficient version keeps only in shared memory and
recomputes in the backward pass (quadratic -> linear memory, at 15-20 %
more time in the README's measurement).

This builds the same architecture with random weights and a random
CIFAR-sized batch (no dataset): DenseNet-BC, growth 12, depth 100 (three
dense blocks of 16 bottleneck layers), compression 0.5.  Both networks share
everything except the bottleneck's first stage:

    plain:      torch.cat -> BatchNorm (batch statistics) -> ReLU -> conv 1x1
    efficient:  dense.EfficientBottleneckStage (shared buffer + recompute on
                libmeswish's kernels) -> conv 1x1 inside the same function

and report the bytes held after the forward, the peak over a training step,
the step time, and the agreement of loss and gradients.

    python -m memory_efficient_activation_amd.dense_experiment [--depth 100] [--batch 64] [--graph]
"""

from __future__ import annotations

import argparse
import json
import time

import torch
import torch.nn as nn
import torch.nn.functional as F

from . import dense


class DenseLayer(nn.Module):
    def __init__(self, in_channels: int, growth: int, efficient: bool, shared):
        super().__init__()
        inner = 4 * growth
        self.efficient = efficient
        self.stage1 = (dense.EfficientBottleneckStage(in_channels, inner, shared) if efficient
                       else dense.NaiveBottleneckStage(in_channels, inner))
        self.bn2 = nn.BatchNorm2d(inner)
        self.conv2 = nn.Conv2d(inner, growth, 3, padding=1, bias=False)

    def forward(self, feats, stats):
        h = self.stage1(feats, stats) if self.efficient else self.stage1(feats)
        return self.conv2(F.relu(self.bn2(h)))


class DenseBlock(nn.Module):
    def __init__(self, layers: int, in_channels: int, growth: int, efficient: bool, shared):
        super().__init__()
        self.efficient, self.shared = efficient, shared
        self.layers = nn.ModuleList(
            DenseLayer(in_channels + i * growth, growth, efficient, shared) for i in range(layers))

    def forward(self, x):
        feats = [x]
        # Each feature map's batch statistics, computed once when it is made.
        stats = [dense.bn_stats(x, self.shared)] if self.efficient else None
        for layer in self.layers:
            y = layer(feats, stats)
            feats.append(y)
            if self.efficient:
                stats.append(dense.bn_stats(y, self.shared))
        return torch.cat(feats, dim=1)


class Transition(nn.Sequential):
    def __init__(self, cin: int, cout: int):
        super().__init__(nn.BatchNorm2d(cin), nn.ReLU(), nn.Conv2d(cin, cout, 1, bias=False),
                         nn.AvgPool2d(2))


class DenseNetBC(nn.Module):
    """DenseNet-BC for 32 x 32 inputs (the README's CIFAR configuration)."""

    def __init__(self, depth: int = 100, growth: int = 12, efficient: bool = True,
                 num_classes: int = 10):
        super().__init__()
        per_block = (depth - 4) // 6
        self.shared = dense.SharedBuffer() if efficient else None
        c = 2 * growth
        mods = [nn.Conv2d(3, c, 3, padding=1, bias=False)]
        for b in range(3):
            mods.append(DenseBlock(per_block, c, growth, efficient, self.shared))
            c += per_block * growth
            if b < 2:
                mods.append(Transition(c, c // 2))
                c //= 2
        self.features = nn.Sequential(*mods)
        self.norm = nn.BatchNorm2d(c)
        self.fc = nn.Linear(c, num_classes)

    def forward(self, x):
        h = F.relu(self.norm(self.features(x)))
        return self.fc(F.adaptive_avg_pool2d(h, 1).flatten(1))


def _requested(kind="current") -> int:
    return int(torch.cuda.memory_stats()[f"requested_bytes.all.{kind}"])


def _step(model, x, y):
    base = _requested()
    loss = F.cross_entropy(model(x), y)
    torch.cuda.synchronize()
    retained = _requested() - base
    loss.backward()
    torch.cuda.synchronize()
    return float(loss), retained


def measure(depth: int = 100, batch: int = 64, growth: int = 12, reps: int = 5,
            seed: int = 0) -> dict:
    dev = torch.device("cuda")
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(batch, 3, 32, 32, generator=g).to(dev)
    y = torch.randint(0, 10, (batch,), generator=g).to(dev)
    torch.manual_seed(seed)
    plain = DenseNetBC(depth, growth, efficient=False).to(dev)
    eff = DenseNetBC(depth, growth, efficient=True).to(dev)
    # Same weights: the efficient stage names its BN parameters gamma/beta.
    with torch.no_grad():
        pe = dict(eff.named_parameters())
        for name, p in plain.named_parameters():
            pe[name].copy_(p)
    out = {"model": f"DenseNet-BC-{depth}, growth {growth}", "batch": batch, "input": "32x32x3",
           "dtype": "float32"}
    grads = {}
    for name, model in (("naive", plain), ("memory_efficient", eff)):
        model.train()
        for _ in range(2):  # warm up the convolution libraries
            model.zero_grad(set_to_none=True)
            _step(model, x, y)
        model.zero_grad(set_to_none=True)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = _requested()
        loss, retained = _step(model, x, y)
        peak = _requested("peak") - base
        grads[name] = {k: p.grad.detach().clone() for k, p in model.named_parameters()}
        times = []
        for _ in range(reps):
            model.zero_grad(set_to_none=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            _step(model, x, y)
            times.append(time.perf_counter() - t0)
        out[name] = {"retained_after_forward_bytes": retained, "peak_step_bytes": peak,
                     "step_ms": round(1e3 * sorted(times)[len(times) // 2], 3), "loss": loss}
    nv, ef = out["naive"], out["memory_efficient"]
    out["retained_saved_fraction"] = round(1 - ef["retained_after_forward_bytes"]
                                           / nv["retained_after_forward_bytes"], 4)
    out["peak_saved_fraction"] = round(1 - ef["peak_step_bytes"] / nv["peak_step_bytes"], 4)
    out["time_ratio_efficient_over_naive"] = round(ef["step_ms"] / nv["step_ms"], 4)
    out["rel_loss_diff"] = abs(ef["loss"] - nv["loss"]) / abs(nv["loss"])
    out["max_rel_grad_diff"] = max(
        float((grads["memory_efficient"][k] - grads["naive"][k]).abs().max()
              / grads["naive"][k].abs().max().clamp_min(1e-30)) for k in grads["naive"])
    out["shared_buffer_bytes"] = eff.shared.nbytes
    # The stored maps the method removes: per bottleneck, the concatenation
    # and its normalized (ReLU) form, each C_l x batch x H x W binary32.
    per_block = (depth - 4) // 6
    c, side, quad = 2 * growth, 32, 0
    for b in range(3):
        for i in range(per_block):
            quad += 2 * (c + i * growth) * batch * side * side * 4
        c = (c + per_block * growth) // 2
        side //= 2
    out["concat_and_bn_maps_bytes"] = quad
    return out


def measure_graph(depth: int = 100, batch: int = 64, growth: int = 12, reps: int = 20,
                  checks: int = 3, seed: int = 0) -> dict:
    """The same training step (forward + backward) of both networks captured
    once into a HIP graph and replayed: the step's GPU time without the
    host's per-layer launch cost.  Every checked replay, with eager work and
    synchronisations between replays, is compared with an eager step on the
    same weights and batch (loss and every parameter's gradient)."""
    dev = torch.device("cuda")
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(batch, 3, 32, 32, generator=g).to(dev)
    y = torch.randint(0, 10, (batch,), generator=g).to(dev)
    torch.manual_seed(seed)
    plain = DenseNetBC(depth, growth, efficient=False).to(dev)
    eff = DenseNetBC(depth, growth, efficient=True).to(dev)
    with torch.no_grad():
        pe = dict(eff.named_parameters())
        for name, p in plain.named_parameters():
            pe[name].copy_(p)
    out = {"model": f"DenseNet-BC-{depth}, growth {growth}", "batch": batch, "dtype": "float32",
           "replays_timed": reps, "replays_checked": checks}
    for name, model in (("naive", plain), ("memory_efficient", eff)):
        model.train()
        model.zero_grad(set_to_none=True)
        ref_loss = F.cross_entropy(model(x), y)
        ref_loss.backward()
        ref_loss = float(ref_loss.detach())
        ref = {k: p.grad.detach().clone() for k, p in model.named_parameters()}
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up on a side stream, as capture requires
            for _ in range(3):
                model.zero_grad(set_to_none=True)
                F.cross_entropy(model(x), y).backward()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        model.zero_grad(set_to_none=True)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            static_loss = F.cross_entropy(model(x), y)
            static_loss.backward()
        worst_loss, worst_grad = 0.0, 0.0
        for _ in range(checks):
            graph.replay()
            torch.cuda.synchronize()
            worst_loss = max(worst_loss, abs(float(static_loss) - ref_loss) / abs(ref_loss))
            for k, p in model.named_parameters():
                worst_grad = max(worst_grad, float((p.grad - ref[k]).abs().max()
                                                   / ref[k].abs().max().clamp_min(1e-30)))
            torch.randn(1 << 20, device=dev).sum().item()  # eager work between replays
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        graph.replay()
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        out[name] = {"graph_step_ms": round(a.elapsed_time(b) / reps, 3),
                     "replay_vs_eager_loss_rel": worst_loss,
                     "replay_vs_eager_grad_rel": worst_grad}
        del graph
    out["graph_time_ratio_efficient_over_naive"] = round(
        out["memory_efficient"]["graph_step_ms"] / out["naive"]["graph_step_ms"], 4)
    return out


def errors_vs_binary64(depth: int = 40, batch: int = 16, growth: int = 12, seed: int = 0) -> dict:
    """Per-parameter gradient error of the plain and the efficient network on
    the GPU against the plain network evaluated in binary64 on the CPU (same
    weights and batch): max |g - g64| / max |g64| per parameter, and the
    loss error.  The binary64 CPU network runs only torch's own CPU ops."""
    import copy
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(batch, 3, 32, 32, generator=g)
    y = torch.randint(0, 10, (batch,), generator=g)
    torch.manual_seed(seed)
    plain = DenseNetBC(depth, growth, efficient=False)
    eff = DenseNetBC(depth, growth, efficient=True)
    with torch.no_grad():
        pe = dict(eff.named_parameters())
        for name, p in plain.named_parameters():
            pe[name].copy_(p)
    ref = copy.deepcopy(plain).double()
    loss64 = F.cross_entropy(ref(x.double()), y)
    loss64.backward()
    g64 = {k: p.grad for k, p in ref.named_parameters()}
    dev = torch.device("cuda")
    out = {"loss64": float(loss64)}
    for name, model in (("naive", plain), ("memory_efficient", eff)):
        model = model.to(dev)
        loss = F.cross_entropy(model(x.to(dev)), y.to(dev))
        loss.backward()
        torch.cuda.synchronize()
        out[name] = {"loss_rel_err": abs(float(loss) - float(loss64)) / abs(float(loss64)),
                     "grad_rel_err": {k: float((p.grad.double().cpu() - g64[k]).abs().max()
                                               / g64[k].abs().max())
                                      for k, p in model.named_parameters()}}
    return out


def main():
    p = argparse.ArgumentParser(description=__doc__,
                                formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--depth", type=int, default=100)
    p.add_argument("--batch", type=int, default=64)
    p.add_argument("--reps", type=int, default=5)
    p.add_argument("--graph", action="store_true",
                   help="also time the step captured into a HIP graph (replays checked)")
    a = p.parse_args()
    print(json.dumps(measure(a.depth, a.batch, reps=a.reps)), flush=True)
    if a.graph:
        print(json.dumps(measure_graph(a.depth, a.batch)), flush=True)


if __name__ == "__main__":
    main()
