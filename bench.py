#!/usr/bin/env python3
"""Benchmark: memory-efficient Swish forward + backward on one MI355X.

Workload: the transformer-scale activation of "What activations cost, in
memory and in arithmetic" (Given; Step 1): bfloat16 [8, 2048, 4096] =
67,108,864 elements, alpha 1.0, x ~ N(0,1) (seed 0), dy ~ 0.01 N(0,1)
(seed 1), inputs resident in HBM before timing starts.

One step = one forward launch (read x, write y) + one backward launch (read
x and dy, write dx) through the C ABI of libmeswish.  Algorithmic bytes per
step = 2 b n + 3 b n = 671,088,640 B (b = 2).  The timed region is K steps
back to back between two device synchronisations; ``value`` is algorithmic
bytes over wall time, in decimal GB/s.  Four copies of the buffers are used
in rotation so that no kernel can read its inputs from the 256 MB Infinity
Cache: every counted byte crosses the HBM interface.

Also reported (one JSON line on stdout):
  roofline      the dominant kernel (the backward): algorithmic bytes per
                launch / mean launch time, from HIP events on the launch
                stream around K back-to-back backward launches (same
                rotation), against 8 TB/s;
                ``traffic`` = HBM bytes per launch from rocprofv3 counters
                (profiles/), or null if the kernel source changed since.
  cpu_baseline  the CPU oracle (binary64 C, all host cores) on the same
                workload, same algorithmic bytes.
  copy_ceiling  a plain 16-byte copy kernel (read one tensor, write one).
  bytes_retained  bytes kept for the backward: x only, vs 3 maps (naive).

``--act KIND`` measures another activation of the family of the same page
(relu, leaky_relu, sigmoid, tanh, gelu, gelu_tanh) on the same workload;
``--act all`` prints one line per activation, Swish first.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "HBM GB/s + fraction of peak, Swish fwd+bwd, 67M-elem bf16, 1 MI355X"
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD public specification
KERNEL_SOURCES = [os.path.join(ROOT, "memory_efficient_activation_amd", "csrc", f)
                  for f in ("meswish.hip", "act_math.h")]
SETS = 4
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "swish_bwd_bf16_8x2048x4096_traffic.md")
FAMILY = ["swish", "relu", "leaky_relu", "sigmoid", "tanh", "gelu", "gelu_tanh"]
ORACLE_NAME = {"gelu": "gelu_erf"}
# Flops per element of each activation as "What activations cost, in memory
# and in arithmetic" (Given) counts them, forward; Swish is sigmoid + 2.
PAGE_FLOPS = {"swish": 6, "relu": 1, "leaky_relu": 2, "sigmoid": 4, "tanh": 6, "gelu": 12,
              "gelu_tanh": 8}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--act", default="swish", choices=FAMILY + ["all"],
                   help="activation to measure (default swish, the headline)")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the CPU oracle timing (profiling runs)")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the copy-ceiling measurement")
    p.add_argument("--cpu-reps", type=int, default=3)
    return p.parse_args()


def source_sha256() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profile():
    """HBM bytes per backward launch measured by rocprofv3 counters, if the
    committed summary was taken on the current kernel sources."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None, "no counter summary"
    text = open(TRAFFIC_PROFILE).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_b):
        return None, "counter summary unreadable"
    if m_sha.group(1) != source_sha256():
        return None, "kernel changed since counters were taken"
    return float(m_b.group(1)), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


class Rig:
    """The workload on the device: SETS copies of (x, dy, y, dx)."""

    def __init__(self, torch, w, dev):
        self.torch = torch
        self.n = w.numel

        def to_dev(a):
            return torch.from_numpy(a).view(torch.int16).view(torch.bfloat16).to(dev)

        # Kernel number k (forward and backward alternate) uses set k % SETS,
        # so no kernel reads memory that any of the previous SETS - 1 kernels
        # touched (>= 800 MB of traffic, three times the 256 MB Infinity
        # Cache): every input byte comes from HBM.
        x0, dy0 = to_dev(w.xs[0]), to_dev(w.dys[0])
        self.bufs = []
        for _ in range(SETS):
            xs, dys = x0.clone(), dy0.clone()
            self.bufs.append((xs, dys, torch.empty_like(xs), torch.empty_like(xs)))
        del x0, dy0
        self.ptrs = [tuple(t.data_ptr() for t in b) for b in self.bufs]
        self.stream = torch.cuda.current_stream(dev)
        self.sh = self.stream.cuda_stream

    def region(self, fn, count):
        """count calls of fn(i) between two events on the launch stream."""
        torch = self.torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(self.stream)
        for i in range(count):
            fn(i)
        b.record(self.stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, a.elapsed_time(b)


def measure(args, act, rig, w, lib, torch):
    from memory_efficient_activation_amd import _lib, accounting

    n, dtype = w.numel, w.dtype
    param = w.alpha if act == "swish" else _lib.DEFAULT_PARAM.get(act, 0.0)
    code, dt = _lib.ACTS[act], _lib.BF16
    ptrs, sh = rig.ptrs, rig.sh

    def fwd(j):
        xp, _, yp, _ = ptrs[j % SETS]
        _lib.check(lib.meswish_act_fwd(code, xp, yp, n, param, dt, sh), "meswish_act_fwd")

    def bwd(j):
        xp, dyp, _, dxp = ptrs[j % SETS]
        _lib.check(lib.meswish_act_bwd(code, xp, dyp, dxp, n, param, dt, sh), "meswish_act_bwd")

    def step(i):
        fwd(2 * i)
        bwd(2 * i + 1)

    fwd_b = accounting.fwd_bytes(n, dtype)
    bwd_b = accounting.bwd_bytes(n, dtype)
    step_b = fwd_b + bwd_b

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    wall, gpu_ms = rig.region(step, K)
    log(f"[bench] {act}: timed {K} steps: wall {wall * 1e3:.2f} ms, events {gpu_ms:.2f} ms")
    # Per-kernel launch durations: each kernel alone, back to back on the
    # rotating sets, between two events on the launch stream.
    _, bwd_total = rig.region(bwd, K)
    _, fwd_total = rig.region(fwd, K)
    bwd_us, fwd_us = bwd_total * 1e3 / K, fwd_total * 1e3 / K
    bwd_gbps = bwd_b / (bwd_us * 1e-6) / 1e9
    fwd_gbps = fwd_b / (fwd_us * 1e-6) / 1e9
    value = step_b * K / wall / 1e9
    headline = act == "swish"
    traffic, traffic_note = traffic_from_profile() if headline else (None, "counters taken for Swish")

    result = {
        "metric": METRIC if headline else
        f"HBM GB/s + fraction of peak, {act} fwd+bwd, 67M-elem bf16, 1 MI355X",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{act} fwd+bwd, bf16 [8,2048,4096] (67,108,864 elements)"
                               + (", alpha=1.0" if headline else ""),
                   "n": n, "param": param, "bytes_per_step": step_b,
                   "x": "N(0,1) seed 0", "dy": "0.01*N(0,1) seed 1", "buffer_sets": SETS},
        "frac_peak": round(value / PEAK_HBM_GBPS, 4),
        "elements_per_s": round(n * K / wall, 1),
        "gpu_ms_per_step_events": round(gpu_ms / K, 5),
        "fwd": {"bytes": fwd_b, "mean_us": round(fwd_us, 2), "GBps": round(fwd_gbps, 1)},
        "bwd": {"bytes": bwd_b, "mean_us": round(bwd_us, 2), "GBps": round(bwd_gbps, 1)},
        "roofline": {"kernel": f"act_vec_kernel<bf16, bwd, {act}>", "bound": "hbm",
                     "achieved": round(bwd_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(bwd_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "traffic_note": traffic_note,
                     "bytes_per_launch": bwd_b, "mean_launch_us": round(bwd_us, 2),
                     "page_flops_per_element_fwd": PAGE_FLOPS[act]},
        "bytes_retained": {"memory_efficient": accounting.retained_bytes(n, dtype),
                           "naive_3_maps": accounting.retained_bytes(n, dtype, naive=True)},
    }

    if not args.no_extras:
        def copy(j):
            xp, _, yp, _ = ptrs[j % SETS]
            _lib.check(lib.meswish_copy(xp, yp, 2 * n, sh), "meswish_copy")
        for i in range(5):
            copy(i)
        _, cms = rig.region(copy, K)
        copy_us = cms * 1e3 / K
        copy_gbps = 2 * (2 * n) / (copy_us * 1e-6) / 1e9
        result["copy_ceiling"] = {"bytes": 4 * n, "mean_us": round(copy_us, 2),
                                  "GBps": round(copy_gbps, 1),
                                  "bwd_frac_of_copy": round(bwd_gbps / copy_gbps, 4),
                                  "value_frac_of_copy": round(value / copy_gbps, 4)}

    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.Oracle()
        threads = len(os.sched_getaffinity(0))
        oname = ORACLE_NAME.get(act, act)
        times = []
        for _ in range(max(1, args.cpu_reps)):
            c0 = time.perf_counter()
            orc.act_fwd(oname, w.xs[0], param, threads=threads)
            orc.act_bwd(oname, w.xs[0], w.dys[0], param, threads=threads, want_scale=False)
            times.append(time.perf_counter() - c0)
        ct = statistics.median(times)
        result["cpu_baseline"] = {"value": round(step_b / ct / 1e9, 3), "unit": "GB/s",
                                  "cores": threads, "kind": "oracle",
                                  "sample": f"the full workload ({n} elements) fwd+bwd, binary64 C "
                                            f"oracle, median of {len(times)} runs ({ct:.2f} s each)",
                                  "elements_per_s": round(n / ct, 1)}
        log(f"[bench] {act}: cpu baseline {ct:.2f} s with {threads} threads")
    return result


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the Swish path is element-wise and would shard "
              "with no communication (each GPU runs its local tensor); multi-GPU runs are not "
              "part of this build. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from memory_efficient_activation_amd import _lib, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a HIP GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = _lib.library()

    t_gen = time.perf_counter()
    w = inputs.make(3)
    log(f"[bench] inputs generated in {time.perf_counter() - t_gen:.1f} s: {w.name}, n={w.numel}")
    rig = Rig(torch, w, dev)
    acts = FAMILY if args.act == "all" else [args.act]
    for act in acts:
        print(json.dumps(measure(args, act, rig, w, lib, torch)), flush=True)


if __name__ == "__main__":
    main()
