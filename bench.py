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
KERNEL_SOURCE = os.path.join(ROOT, "memory_efficient_activation_amd", "csrc", "meswish.hip")
SETS = 4
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "swish_bwd_bf16_8x2048x4096_traffic.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the CPU oracle timing (profiling runs)")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the copy-ceiling measurement")
    p.add_argument("--cpu-reps", type=int, default=3)
    return p.parse_args()


def source_sha256() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_from_profile():
    """HBM bytes per backward launch measured by rocprofv3 counters, if the
    committed summary was taken on the current kernel source."""
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


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the Swish path is element-wise and would shard "
              "with no communication (each GPU runs its local tensor); multi-GPU runs are not "
              "part of this build. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from memory_efficient_activation_amd import _lib, accounting, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a HIP GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = _lib.library()

    t_gen = time.perf_counter()
    w = inputs.make(3)
    n, dtype, alpha = w.numel, w.dtype, w.alpha
    log(f"[bench] inputs generated in {time.perf_counter() - t_gen:.1f} s: {w.name}, n={n}")

    def to_dev(a):
        return torch.from_numpy(a).view(torch.int16).view(torch.bfloat16).to(dev)

    # SETS copies of (x, dy, y, dx).  Kernel number k (forward and backward
    # alternate) uses set k % SETS, so no kernel reads memory that any of
    # the previous SETS - 1 kernels touched (>= 800 MB of traffic, three
    # times the 256 MB Infinity Cache): every input byte comes from HBM.
    x0, dy0 = to_dev(w.xs[0]), to_dev(w.dys[0])
    bufs = []
    for _ in range(SETS):
        xs, dys = x0.clone(), dy0.clone()
        bufs.append((xs, dys, torch.empty_like(xs), torch.empty_like(xs)))
    del x0, dy0
    ptrs = [tuple(t.data_ptr() for t in b) for b in bufs]
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    code = _lib.BF16

    fwd_b = accounting.fwd_bytes(n, dtype)
    bwd_b = accounting.bwd_bytes(n, dtype)
    step_b = fwd_b + bwd_b

    def fwd(j):
        xp, _, yp, _ = ptrs[j % SETS]
        _lib.check(lib.swish_fwd(xp, yp, n, alpha, code, sh), "swish_fwd")

    def bwd(j):
        xp, dyp, _, dxp = ptrs[j % SETS]
        _lib.check(lib.swish_bwd(xp, dyp, dxp, n, alpha, code, sh), "swish_bwd")

    def step(i):
        fwd(2 * i)
        bwd(2 * i + 1)

    def region(fn, count):
        """count calls of fn(i) between two events on the launch stream."""
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        for i in range(count):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, a.elapsed_time(b)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    K = args.steps
    wall, gpu_ms = region(step, K)
    log(f"[bench] timed {K} steps: wall {wall * 1e3:.2f} ms, events {gpu_ms:.2f} ms")

    # Per-kernel launch durations: each kernel alone, back to back on the
    # rotating sets, between two events on the launch stream.
    _, bwd_total = region(bwd, K)
    _, fwd_total = region(fwd, K)
    bwd_us = bwd_total * 1e3 / K
    fwd_us = fwd_total * 1e3 / K
    bwd_gbps = bwd_b / (bwd_us * 1e-6) / 1e9
    fwd_gbps = fwd_b / (fwd_us * 1e-6) / 1e9

    ms_per_step = wall * 1e3 / K
    value = step_b * K / wall / 1e9
    traffic, traffic_note = traffic_from_profile()

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "swish fwd+bwd, bf16 [8,2048,4096] (67,108,864 elements), alpha=1.0",
                   "n": n, "alpha": alpha, "bytes_per_step": step_b,
                   "x": "N(0,1) seed 0", "dy": "0.01*N(0,1) seed 1",
                   "buffer_sets": SETS},
        "frac_peak": round(value / PEAK_HBM_GBPS, 4),
        "elements_per_s": round(n * K / wall, 1),
        "gpu_ms_per_step_events": round(gpu_ms / K, 5),
        "fwd": {"bytes": fwd_b, "mean_us": round(fwd_us, 2), "GBps": round(fwd_gbps, 1)},
        "bwd": {"bytes": bwd_b, "mean_us": round(bwd_us, 2), "GBps": round(bwd_gbps, 1)},
        "roofline": {"kernel": "swish_vec_kernel<bf16, bwd>", "bound": "hbm",
                     "achieved": round(bwd_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(bwd_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "traffic_note": traffic_note,
                     "bytes_per_launch": bwd_b, "mean_launch_us": round(bwd_us, 2)},
        "bytes_retained": {"memory_efficient": accounting.retained_bytes(n, dtype),
                           "naive_3_maps": accounting.retained_bytes(n, dtype, naive=True)},
    }

    if not args.no_extras:
        # Plain 16-byte copy of one tensor (read b n, write b n), same rotation.
        def copy(j):
            xp, _, yp, _ = ptrs[j % SETS]
            _lib.check(lib.meswish_copy(xp, yp, 2 * n, sh), "meswish_copy")
        for i in range(5):
            copy(i)
        _, cms = region(copy, K)
        copy_us = cms * 1e3 / K
        copy_gbps = 2 * (2 * n) / (copy_us * 1e-6) / 1e9
        result["copy_ceiling"] = {"bytes": 4 * n, "mean_us": round(copy_us, 2),
                                  "GBps": round(copy_gbps, 1),
                                  "bwd_frac_of_copy": round(bwd_gbps / copy_gbps, 4),
                                  "value_frac_of_copy": round(value / copy_gbps, 4)}
        log(f"[bench] copy ceiling {copy_gbps:.0f} GB/s")

    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.Oracle()
        threads = len(os.sched_getaffinity(0))
        times = []
        for _ in range(max(1, args.cpu_reps)):
            c0 = time.perf_counter()
            orc.fwd(w.xs[0], alpha, threads=threads)
            orc.bwd(w.xs[0], w.dys[0], alpha, threads=threads, want_scale=False)
            times.append(time.perf_counter() - c0)
        ct = statistics.median(times)
        result["cpu_baseline"] = {"value": round(step_b / ct / 1e9, 3), "unit": "GB/s",
                                  "cores": threads, "kind": "oracle",
                                  "sample": f"the full workload ({n} elements) fwd+bwd, binary64 C oracle, "
                                            f"median of {len(times)} runs ({ct:.2f} s each)",
                                  "elements_per_s": round(n / ct, 1)}
        log(f"[bench] cpu baseline {ct:.2f} s with {threads} threads")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
