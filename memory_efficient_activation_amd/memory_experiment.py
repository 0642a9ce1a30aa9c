"""Module-level memory experiment: naive vs memory-efficient activations.

The blog post "Memory efficient Swish" measures GPU memory of EfficientNets
with the plain and the memory-efficient Swish ("How much GPU memory is
saved?"; its tables are lost in extraction) and explains the saving in "Why
simple Swish implementation is inefficient?": the plain module keeps three
feature maps for the backward -- its input, the sigmoid and the product --
where the memory-efficient one keeps only its input.

This experiment reproduces the shape of that measurement without model
weights or data.  A synthetic network is a set of chains; each chain repeats
the block

    z -> h = w * z   (per-channel scale: stands in for the producing layer,
                      which keeps its own input z, as a convolution would)
      -> a = act(h)  (the activation under test; a feeds the next block)

and the loss is the sum of the last outputs times fixed random weights.
Activation memory retained after the forward is, per block:

    memory-efficient:  z (kept by the scale) + h (kept by the activation)
    plain Swish:       z + h + sigmoid(h)   (the product a is the next z)

so the efficient network keeps one feature map less per activation (the
sigmoid map; the product is kept by its consumer in both).  With bfloat16
storage both networks are also compared with the plain network evaluated
in binary32 on the same inputs.  The
script measures the bytes requested by live tensors (retained after the
forward, peak over the step) and the step time, and checks that both networks give the
same loss and gradients.

    python -m memory_efficient_activation_amd.memory_experiment --workload efficientnet
    python -m memory_efficient_activation_amd.memory_experiment --workload transformer
"""

from __future__ import annotations

import argparse
import json
import time

import torch

from .inputs import EFFICIENTNET_MBCONV_SHAPES
from .module import MemoryEfficientSwish
from .naive import Swish

WORKLOADS = {
    # The seven NHWC activation shapes at batch 32 of the grouped workload,
    # two blocks each.
    "efficientnet": {"shapes": EFFICIENTNET_MBCONV_SHAPES, "blocks": 2},
    # "What activations cost, in memory and in arithmetic" (Given): one
    # [8, 2048, 4096] activation per layer over L = 32 layers.
    "transformer": {"shapes": [(8, 2048, 4096)], "blocks": 32},
}


def build(shapes, blocks, dtype, device, seed=0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    chains = []
    for shape in shapes:
        c = shape[-1]
        x = torch.randn(*shape, generator=g).to(dtype).to(device)
        ws = [(1.0 + 0.1 * torch.randn(c, generator=g)).to(dtype).to(device).requires_grad_(True)
              for _ in range(blocks)]
        r = torch.randn(*shape, generator=g).to(dtype).to(device)
        chains.append((x, ws, r))
    return chains


def _requested(kind: str = "current") -> int:
    """Bytes the live tensors asked for (the caching allocator's block
    rounding and unsplit cached blocks excluded)."""
    return int(torch.cuda.memory_stats()[f"requested_bytes.all.{kind}"])


def run_step(chains, make_act):
    """One forward + backward; returns (loss, bytes retained after forward)."""
    base = _requested()
    loss = 0.0
    for x, ws, r in chains:
        z = x
        for w in ws:
            z = make_act()(z * w)
        loss = loss + (z * r).sum(dtype=torch.float32)
    torch.cuda.synchronize()
    retained = _requested() - base
    loss.backward()
    torch.cuda.synchronize()
    return loss.detach(), retained


def measure(workload: str, dtype=torch.bfloat16, alpha: float = 1.0, reps: int = 3) -> dict:
    spec = WORKLOADS[workload]
    dev = torch.device("cuda")
    chains = build(spec["shapes"], spec["blocks"], dtype, dev)
    n_act = sum(int(torch.tensor(s).prod()) for s in spec["shapes"]) * spec["blocks"]
    esize = torch.empty((), dtype=dtype).element_size()
    out = {"workload": workload, "dtype": str(dtype).replace("torch.", ""),
           "activations": len(spec["shapes"]) * spec["blocks"],
           "activation_elements": n_act, "one_map_per_activation_bytes": n_act * esize}
    grads = {}
    for name, make in (("naive", lambda: Swish(alpha)),
                       ("memory_efficient", lambda: MemoryEfficientSwish(alpha))):
        for _, ws, _ in chains:
            for w in ws:
                w.grad = None
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = _requested()
        loss, retained = run_step(chains, make)
        peak = _requested("peak") - base
        grads[name] = [w.grad.float().clone() for _, ws, _ in chains for w in ws]
        times = []
        for _ in range(reps):
            for _, ws, _ in chains:
                for w in ws:
                    w.grad = None
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            run_step(chains, make)
            times.append(time.perf_counter() - t0)
        out[name] = {"retained_after_forward_bytes": int(retained), "peak_step_bytes": int(peak),
                     "step_ms": round(1e3 * sorted(times)[len(times) // 2], 3),
                     "loss": float(loss)}
    if dtype != torch.float32:
        # Reference: the plain network in binary32 on the same (upcast)
        # inputs and weights; both bfloat16 networks are compared with it.
        ref_chains = [(x.float(), [w.detach().float().requires_grad_(True) for w in ws], r.float())
                      for x, ws, r in chains]
        ref_loss, _ = run_step(ref_chains, lambda: Swish(alpha))
        ref_grads = [w.grad for _, ws, _ in ref_chains for w in ws]
        for name in ("naive", "memory_efficient"):
            out[name]["loss_rel_err_vs_f32"] = abs(out[name]["loss"] - float(ref_loss)) / abs(float(ref_loss))
            out[name]["grad_rel_err_vs_f32"] = max(
                float((a - b).abs().max() / b.abs().max().clamp_min(1e-30))
                for a, b in zip(grads[name], ref_grads))
        del ref_chains, ref_grads
    nv, ef = out["naive"], out["memory_efficient"]
    out["retained_saved_bytes"] = nv["retained_after_forward_bytes"] - ef["retained_after_forward_bytes"]
    out["retained_saved_fraction"] = round(out["retained_saved_bytes"] / nv["retained_after_forward_bytes"], 4)
    out["peak_saved_fraction"] = round(1 - ef["peak_step_bytes"] / nv["peak_step_bytes"], 4)
    out["max_rel_grad_diff"] = max(float(((a - b).abs().max() / b.abs().max().clamp_min(1e-30)))
                                   for a, b in zip(grads["memory_efficient"], grads["naive"]))
    out["rel_loss_diff"] = abs(ef["loss"] - nv["loss"]) / max(abs(nv["loss"]), 1e-30)
    return out


def main():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--workload", choices=sorted(WORKLOADS), default="efficientnet")
    p.add_argument("--dtype", choices=["bf16", "f32"], default="bf16")
    a = p.parse_args()
    dtype = torch.bfloat16 if a.dtype == "bf16" else torch.float32
    print(json.dumps(measure(a.workload, dtype)), flush=True)


if __name__ == "__main__":
    main()
