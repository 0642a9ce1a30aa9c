#!/usr/bin/env python3
"""Benchmark: memory-efficient Swish forward + backward on one MI355X.

Workload: the transformer-scale activation of "What activations cost, in
memory and in arithmetic" (Given; Step 1): bfloat16 [8, 2048, 4096] =
67,108,864 elements, alpha 1.0, x ~ N(0,1) (seed 0), dy ~ 0.01 N(0,1)
(seed 1), inputs resident in HBM before timing starts.

One step = one forward launch (read x, write y) + one backward launch (read
x and dy, write dx) through the C ABI of libmeswish.  Algorithmic bytes per
step = 2 b n + 3 b n = 671,088,640 B (b = 2).  W untimed steps come first
(default 500, about 50 ms): for some 20 ms after a sustained load starts,
the GPU's clocks dip and recover, and the timed region is meant to measure
the sustained rate.  The timed region is K steps back to back between two
device synchronisations; ``value`` is algorithmic
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
                workload, same algorithmic bytes; runs repeat until
                --cpu-seconds (10 s) have passed, and the median run counts.
  copy_ceiling  a plain 16-byte copy kernel (read one tensor, write one).
  bytes_retained  bytes kept for the backward: x only, vs 3 maps (naive).

``--act KIND`` measures another activation of the family of the same page
(relu, leaky_relu, sigmoid, tanh, gelu, gelu_tanh) on the same workload;
``--act all`` prints one line per activation, Swish first.

``--dense`` measures instead the shared-buffer DenseNet layer stage (README
of efficient_densenet_pytorch, "A memory-efficient implementation of
DenseNets", Motivation) on the widest layer of DenseNet-BC-100's first
block at batch 64 (204 channels of 64 x 32 x 32, the README's Performance
configuration): per training step of that layer, the statistics of its
newest source, the forward, the backward's re-population of the shared
buffer, and the backward (reduction + apply).  ``--dense-dtype`` picks
binary32 (default) or bfloat16 feature maps.

``--grouped`` measures the grouped launch (one kernel per direction) over
the seven EfficientNet MBConv-shaped bf16 tensors of the grouped
configuration, against seven single launches per direction.

``--fft`` measures the FFT convolution layer ("Fast Training of
Convolutional Networks through FFTs") on S=128, f=96, f'=256, n=32, k=7:
one step = forward + input gradient + weight gradient, each transforming
its inputs into one reused frequency buffer, multiplying per frequency
bin, and transforming back.  Reported against PyTorch's direct convolution
(MIOpen) on the same layer.
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
# rocprofv3 counter summaries of the Swish backward, per workload.
TRAFFIC_PROFILES = {
    3: os.path.join(ROOT, "profiles", "swish_bwd_bf16_8x2048x4096_traffic.md"),
    4: os.path.join(ROOT, "profiles", "swish_bwd_f32_8x2048x4096_alpha1.5_traffic.md"),
}
# How each single-tensor workload draws its values (memory_efficient_activation_amd/inputs.py).
RECIPES = {
    1: ("3*N(0,1) seed 0", "N(0,1) seed 1"),
    2: ("N(0,1) seed 0", "N(0,1) seed 1"),
    3: ("N(0,1) seed 0", "0.01*N(0,1) seed 1"),
    4: ("99% N(0,1), 1% +-U(20,90), seed 0", "N(0,1) seed 1"),
}
FAMILY = ["swish", "relu", "leaky_relu", "sigmoid", "tanh", "gelu", "gelu_tanh"]
ORACLE_NAME = {"gelu": "gelu_erf"}
# Flops per element of each activation as "What activations cost, in memory
# and in arithmetic" (Given) counts them, forward; Swish is sigmoid + 2.
PAGE_FLOPS = {"swish": 6, "relu": 1, "leaky_relu": 2, "sigmoid": 4, "tanh": 6, "gelu": 12,
              "gelu_tanh": 8}


def time_cpu(run, args):
    """Repeat run() until at least args.cpu_reps runs and args.cpu_seconds
    of wall time; return (median seconds per run, runs, total seconds)."""
    times = []
    while len(times) < max(1, args.cpu_reps) or sum(times) < args.cpu_seconds:
        c0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - c0)
    return statistics.median(times), len(times), sum(times)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=500,
                   help="untimed steps first (default 500: 25-50 ms of work, past the clock "
                        "transient that follows the start of a sustained load)")
    p.add_argument("--act", default="swish", choices=FAMILY + ["all"],
                   help="activation to measure (default swish, the headline)")
    p.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5],
                   help="Swish workload (default 3, the headline bf16 [8,2048,4096]); "
                        "1, 2 and 4 are the binary32 workloads, 5 the grouped launch")
    p.add_argument("--report", action="store_true",
                   help="per-launch protocol instead: one JSON line per workload and "
                        "direction (median and p10/p90 of scrubbed launches, hot launches, "
                        "copy ceiling, errors against the oracle, band counts, CPU times)")
    p.add_argument("--report-reps", type=int, default=100,
                   help="timed launches per direction in --report (1000 for workload 1)")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the CPU oracle timing (profiling runs)")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the copy-ceiling measurement")
    p.add_argument("--cpu-reps", type=int, default=3,
                   help="least number of timed CPU oracle runs")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="keep repeating the CPU oracle run until this much time has passed")
    p.add_argument("--dense", action="store_true",
                   help="measure the shared-buffer DenseNet layer stage instead")
    p.add_argument("--dense-dtype", default="f32", choices=["f32", "bf16"])
    p.add_argument("--dense-sets", type=int, default=DENSE_SETS,
                   help="rotating buffer sets of the DenseNet layer bench (default 8; fewer "
                        "sets hold less memory but let the caches serve part of the traffic)")
    p.add_argument("--grouped", action="store_true",
                   help="grouped Swish over the 7 EfficientNet-shaped bf16 tensors (config 5)")
    p.add_argument("--fft", action="store_true",
                   help="measure the FFT convolution layer instead")
    return p.parse_args()


def source_sha256() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profile(cfg: int):
    """HBM bytes per backward launch measured by rocprofv3 counters, if the
    committed summary for workload cfg was taken on the current kernel
    sources."""
    path = TRAFFIC_PROFILES.get(cfg)
    if path is None or not os.path.exists(path):
        return None, "no counter summary for this workload"
    text = open(path).read()
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
            t = torch.from_numpy(a)
            if a.dtype.name == "uint16":
                t = t.view(torch.int16).view(torch.bfloat16)
            return t.to(dev)

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

    n, dtype, cfg = w.numel, w.dtype, w.index
    param = w.alpha if act == "swish" else _lib.DEFAULT_PARAM.get(act, 0.0)
    code, dt = _lib.ACTS[act], (_lib.BF16 if dtype == "bf16" else _lib.F32)
    esize = 2 if dtype == "bf16" else 4
    shape = "[" + ",".join(str(d) for d in w.shapes[0]) + "]"
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
    headline = act == "swish" and cfg == 3
    traffic, traffic_note = (traffic_from_profile(cfg) if act == "swish"
                             else (None, "counters taken for Swish"))
    if headline:
        metric = METRIC
    elif cfg == 3:
        metric = f"HBM GB/s + fraction of peak, {act} fwd+bwd, 67M-elem bf16, 1 MI355X"
    else:
        metric = (f"HBM GB/s + fraction of peak, Swish fwd+bwd, {n}-elem {dtype} "
                  f"{shape} alpha={param:g}, 1 MI355X")
    xr, dr = RECIPES[cfg]
    notes = {1: "256 KiB per tensor: the launches are latency-bound and the tensors stay in "
                "the caches (a parity-size workload, not a bandwidth figure)",
             2: "stands in for an EfficientNet stem activation (the blog post's measured "
                "networks are not available)",
             4: "about 0.46 % of the elements take the rare branch (|alpha x| > 86.6)"}

    result = {
        "metric": metric,
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
        "io_dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"{act} fwd+bwd, {dtype} {shape} ({n:,} elements)"
                               + (f", alpha={param:g}" if act == "swish" else ""),
                   "config_index": cfg, "n": n, "param": param, "bytes_per_step": step_b,
                   "x": xr, "dy": dr, "buffer_sets": SETS},
        "frac_peak": round(value / PEAK_HBM_GBPS, 4),
        "elements_per_s": round(n * K / wall, 1),
        "gpu_ms_per_step_events": round(gpu_ms / K, 5),
        "fwd": {"bytes": fwd_b, "mean_us": round(fwd_us, 2), "GBps": round(fwd_gbps, 1)},
        "bwd": {"bytes": bwd_b, "mean_us": round(bwd_us, 2), "GBps": round(bwd_gbps, 1)},
        "roofline": {"kernel": f"act_vec_kernel<{dtype}, bwd, {act}>", "bound": "hbm",
                     "achieved": round(bwd_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(bwd_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "traffic_note": traffic_note,
                     "bytes_per_launch": bwd_b, "mean_launch_us": round(bwd_us, 2),
                     "page_flops_per_element_fwd": PAGE_FLOPS[act]},
        "bytes_retained": {"memory_efficient": accounting.retained_bytes(n, dtype),
                           "naive_3_maps": accounting.retained_bytes(n, dtype, naive=True)},
    }

    if cfg in notes:
        result["config"]["note"] = notes[cfg]
    if not args.no_extras:
        def copy(j):
            xp, _, yp, _ = ptrs[j % SETS]
            _lib.check(lib.meswish_copy(xp, yp, esize * n, sh), "meswish_copy")
        for i in range(5):
            copy(i)
        _, cms = rig.region(copy, K)
        copy_us = cms * 1e3 / K
        copy_gbps = 2 * (esize * n) / (copy_us * 1e-6) / 1e9
        result["copy_ceiling"] = {"bytes": 2 * esize * n, "mean_us": round(copy_us, 2),
                                  "GBps": round(copy_gbps, 1),
                                  "bwd_frac_of_copy": round(bwd_gbps / copy_gbps, 4),
                                  "value_frac_of_copy": round(value / copy_gbps, 4)}

    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.Oracle()
        threads = len(os.sched_getaffinity(0))
        oname = ORACLE_NAME.get(act, act)
        def run():
            orc.act_fwd(oname, w.xs[0], param, threads=threads)
            orc.act_bwd(oname, w.xs[0], w.dys[0], param, threads=threads, want_scale=False)
        ct, runs, total = time_cpu(run, args)
        result["cpu_baseline"] = {"value": round(step_b / ct / 1e9, 3), "unit": "GB/s",
                                  "cores": threads, "kind": "oracle",
                                  "sample": f"the full workload ({n} elements) fwd+bwd, binary64 C "
                                            f"oracle, median of {runs} runs ({ct:.2f} s each, "
                                            f"{total:.1f} s in all)",
                                  "elements_per_s": round(n / ct, 1)}
        log(f"[bench] {act}: cpu baseline {ct:.2f} s x {runs} with {threads} threads")
    return result


DENSE_SETS = 8  # default of --dense-sets
DENSE_SOURCES = [os.path.join(ROOT, "memory_efficient_activation_amd", "csrc", "dense_bn.hip")]


def dense_traffic_from_profile(dtype: str):
    """HBM bytes per forward launch of the DenseNet layer stage from the
    committed rocprofv3 counter summary, if taken on the current source."""
    path = os.path.join(ROOT, "profiles", f"dense_fwd_{dtype}_densenet_bc100_b1l16_traffic.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_b):
        return None, "counter summary unreadable"
    h = hashlib.sha256()
    for f in DENSE_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    if m_sha.group(1) != h.hexdigest():
        return None, "kernel changed since counters were taken"
    return float(m_b.group(1)), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


def measure_dense(args, lib, torch, dev):
    """The DenseNet layer stage: see the module docstring (``--dense``)."""
    from memory_efficient_activation_amd import _lib, dense, dense_inputs as di

    w = di.densenet_bc100_layer(0, di.BLOCK_LAYERS - 1, args.dense_dtype)
    n, hw, C = w.n, w.hw, w.total_channels
    esz = 4 if w.dtype == "f32" else 2
    code = _lib.F32 if w.dtype == "f32" else _lib.BF16
    cmb = C * n * hw * esz                       # one concatenated map, bytes
    new_c = w.channels[-1]                       # the layer's newest source

    def to_dev(a):
        t = torch.from_numpy(a)
        if a.dtype.name == "uint16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(dev)

    gamma, beta = to_dev(w.gamma), to_dev(w.beta)
    sets = []
    xs0 = [to_dev(s_) for s_ in w.sources]
    dz0 = to_dev(w.dz)
    nsets = max(1, args.dense_sets)
    for _ in range(nsets):
        xs = [x.clone() for x in xs0]
        st = [dense.bn_stats(x) for x in xs]
        dxs = [torch.empty_like(x) for x in xs]
        z = torch.empty_like(dz0)
        dz = dz0.clone()
        descs = (_lib.DenseSource * len(xs))(*[
            _lib.DenseSource(x.data_ptr(), d.data_ptr(), t.data_ptr(), int(x.shape[1]), off)
            for x, d, t, off in zip(xs, dxs, st, [sum(w.channels[:j]) for j in range(len(xs))])])
        nbytes = lib.dense_bn_workspace_bytes(n, C, hw)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        ws_new = torch.empty(lib.dense_bn_workspace_bytes(n, new_c, hw), dtype=torch.uint8,
                             device=dev)
        stat_new = torch.empty((new_c, 2), dtype=torch.float64, device=dev)
        dg = torch.empty(C, dtype=torch.float32, device=dev)
        db = torch.empty(C, dtype=torch.float32, device=dev)
        sets.append(dict(xs=xs, st=st, dxs=dxs, z=z, dz=dz, descs=descs, ws=ws, ws_new=ws_new,
                         stat_new=stat_new, dg=dg, db=db))
    del xs0, dz0
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    eps = float(w.eps)
    nsrc = len(w.sources)

    def k_stats(j):
        s_ = sets[j % nsets]
        _lib.check(lib.dense_bn_stats(s_["xs"][-1].data_ptr(), n, new_c, hw, code,
                                      s_["stat_new"].data_ptr(), s_["ws_new"].data_ptr(),
                                      s_["ws_new"].numel(), sh), "dense_bn_stats")

    def k_fwd(j):
        s_ = sets[j % nsets]
        _lib.check(lib.dense_bn_relu_fwd(s_["descs"], nsrc, n, hw, C, gamma.data_ptr(),
                                         beta.data_ptr(), eps, s_["z"].data_ptr(), code, sh),
                   "dense_bn_relu_fwd")

    def k_bwd(j):
        s_ = sets[j % nsets]
        _lib.check(lib.dense_bn_relu_bwd(s_["descs"], nsrc, n, hw, C, gamma.data_ptr(),
                                         beta.data_ptr(), eps, s_["dz"].data_ptr(),
                                         s_["dg"].data_ptr(), s_["db"].data_ptr(),
                                         s_["ws"].data_ptr(), s_["ws"].numel(), code, sh),
                   "dense_bn_relu_bwd")

    def step(i):
        k_stats(4 * i)
        k_fwd(4 * i + 1)
        k_fwd(4 * i + 2)      # the backward's re-population of the shared buffer
        k_bwd(4 * i + 3)

    stats_b, fwd_b, bwd_b = new_c * n * hw * esz, 2 * cmb, 5 * cmb
    step_b = stats_b + 2 * fwd_b + bwd_b

    def region(fn, count):
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
    K = args.steps
    wall, gpu_ms = region(step, K)
    log(f"[bench] dense: timed {K} steps: wall {wall * 1e3:.2f} ms, events {gpu_ms:.2f} ms")
    per = {}
    for name, fn, nb in (("stats", k_stats, stats_b), ("fwd", k_fwd, fwd_b),
                         ("bwd", k_bwd, bwd_b)):
        _, ms = region(fn, K)
        us = ms * 1e3 / K
        per[name] = {"bytes": nb, "mean_us": round(us, 2), "GBps": round(nb / (us * 1e-6) / 1e9, 1)}
    value = step_b * K / wall / 1e9
    # Copy ceiling on one concatenated map's bytes (read + write), same
    # rotation depth; it also calibrates the HBM counters.
    cbufs = [(torch.empty(cmb, dtype=torch.uint8, device=dev),
              torch.empty(cmb, dtype=torch.uint8, device=dev)) for _ in range(max(1, nsets // 2))]

    def k_copy(j):
        a_, b_ = cbufs[j % len(cbufs)]
        _lib.check(lib.meswish_copy(a_.data_ptr(), b_.data_ptr(), cmb, sh), "meswish_copy")

    for i in range(5):
        k_copy(i)
    _, cms = region(k_copy, K)
    copy_us = cms * 1e3 / K
    del cbufs
    traffic, traffic_note = dense_traffic_from_profile(w.dtype)

    # PyTorch's own path on the same layer, for context: torch.cat +
    # batch_norm (training) + relu, forward and autograd backward.
    tx = [x.clone().requires_grad_(True) for x in sets[0]["xs"]]
    tg = gamma.clone().requires_grad_(True)
    tb = beta.clone().requires_grad_(True)
    tdz = sets[0]["dz"]

    def torch_step(_):
        u = torch.cat(tx, dim=1)
        h = torch.relu(torch.nn.functional.batch_norm(u, None, None, tg.to(u.dtype), tb.to(u.dtype),
                                                      training=True, eps=eps))
        h.backward(tdz)

    for i in range(3):
        torch_step(i)
    reps = max(10, K // 10)
    t_wall, _ = region(torch_step, reps)

    result = {
        "metric": f"HBM GB/s + fraction of peak, DenseNet layer stage (concat+BN+ReLU, shared "
                  f"buffer) fwd+recompute+bwd, DenseNet-BC-100 block-1 layer-16 {w.dtype}, "
                  f"1 MI355X",
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
        "io_dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"DenseNet-BC-100 (growth 12) block 1 layer 16 at batch 64: "
                               f"{nsrc} sources, {C} channels of 64x32x32, {w.dtype}",
                   "channels": w.channels, "n": n, "hw": hw, "eps": eps,
                   "bytes_per_step": step_b, "buffer_sets": nsets,
                   "step": "stats(newest source) + fwd + fwd (recompute) + bwd (reduce+apply)"},
        "frac_peak": round(value / PEAK_HBM_GBPS, 4),
        "kernels": per,
        "roofline": {"kernel": f"dense_bn::fwd_kernel<{w.dtype}> (2 launches per step)",
                     "bound": "hbm", "achieved": per["fwd"]["GBps"], "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(per["fwd"]["GBps"] / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "traffic_note": traffic_note,
                     "bytes_per_launch": fwd_b, "mean_launch_us": per["fwd"]["mean_us"]},
        "copy_ceiling": {"bytes": 2 * cmb, "mean_us": round(copy_us, 2),
                         "GBps": round(2 * cmb / (copy_us * 1e-6) / 1e9, 1)},
        "torch_eager_same_layer": {"ms_per_step": round(t_wall * 1e3 / reps, 4),
                                   "note": "torch.cat + batch_norm + relu, fwd + autograd bwd; "
                                           "keeps the concatenation and the output"},
    }
    if not args.no_cpu_baseline:
        import numpy as np
        from oracle import dense_oracle
        from memory_efficient_activation_amd import inputs
        srcs = [inputs.decode(s_).astype(np.float64) for s_ in w.sources]
        dz64 = inputs.decode(w.dz).astype(np.float64)
        def run():
            dense_oracle.forward(srcs, w.gamma, w.beta, eps)
            dense_oracle.backward(srcs, dz64, w.gamma, w.beta, eps)
        ct, runs, total = time_cpu(run, args)
        # The oracle's backward recomputes the forward, as the method does:
        # count the same bytes as one GPU step without the statistics pass.
        cb = 2 * fwd_b + bwd_b
        result["cpu_baseline"] = {"value": round(cb / ct / 1e9, 3), "unit": "GB/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"the full layer ({C} x {n * hw} elements), numpy "
                                            f"binary64 forward + backward, median of {runs} runs "
                                            f"({ct:.2f} s each, {total:.1f} s in all)"}
        log(f"[bench] dense: cpu baseline {ct:.2f} s")
    return result


# Dense binary32 matrix-core (MFMA) throughput of MI355X, AMD's published
# figure.  (The vector ALUs without packed instructions, which the library's
# compile flags disable, give 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz = 78.6.)
PEAK_FP32_MFMA_TFLOPS = 157.3


FFT_SOURCES = [os.path.join(ROOT, "memory_efficient_activation_amd", "csrc", "fft_conv.hip")]


def fft_traffic_from_profile():
    """HBM bytes per launch of the forward's per-bin products, from the
    committed rocprofv3 counter summary, if taken on the current source."""
    path = os.path.join(ROOT, "profiles", "fft_conv_s128_f96_f256_n32_k7_traffic.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_b):
        return None, "counter summary unreadable"
    h = hashlib.sha256()
    for f in FFT_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    if m_sha.group(1) != h.hexdigest():
        return None, "kernel changed since counters were taken"
    return float(m_b.group(1)), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


def measure_fft(args, lib, torch, dev):
    """The FFT convolution layer: see the module docstring (``--fft``)."""
    from memory_efficient_activation_amd import _lib, fft, fft_inputs

    L = fft_inputs.bench_layer()
    S, f, fo, n, k, m = L.S, L.f, L.fo, L.n, L.k, L.m
    P = fft.bins(n)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    x, w, g = (torch.from_numpy(a).to(dev) for a in (L.x, L.w, L.g))
    y = torch.empty((S, fo, m, m), device=dev)
    gx = torch.empty((S, f, n, n), device=dev)
    gw = torch.empty((fo, f, k, k), device=dev)
    fb = lib.fftconv_buffer_bytes(S, f, fo, n)
    freq = torch.empty(fb, dtype=torch.uint8, device=dev)
    fp = freq.data_ptr()

    def op_f(_):
        _lib.check(lib.fftconv_fprop(x.data_ptr(), w.data_ptr(), y.data_ptr(), S, f, fo, n, k, fp,
                                     fb, sh), "fftconv_fprop")

    def op_b(_):
        _lib.check(lib.fftconv_bprop(g.data_ptr(), w.data_ptr(), gx.data_ptr(), S, f, fo, n, k, fp,
                                     fb, sh), "fftconv_bprop")

    def op_a(_):
        _lib.check(lib.fftconv_accgrad(x.data_ptr(), g.data_ptr(), gw.data_ptr(), S, f, fo, n, k,
                                       fp, fb, sh), "fftconv_accgrad")

    def step(i):
        op_f(i)
        op_b(i)
        op_a(i)

    # The forward's stages on the same buffer layout: X, W, then Y.
    sx = fp
    sw = sx + S * f * P * 8
    sy = sw + fo * f * P * 8

    def st_r2c_x(_):
        _lib.check(lib.fftconv_r2c(x.data_ptr(), S * f, n, n, sx, sh), "fftconv_r2c")

    def st_r2c_w(_):
        _lib.check(lib.fftconv_r2c(w.data_ptr(), fo * f, k, n, sw, sh), "fftconv_r2c")

    def st_cmul(_):
        _lib.check(lib.fftconv_cmul(0, sx, sw, sy, S, f, fo, P, sh), "fftconv_cmul")

    def st_c2r(_):
        _lib.check(lib.fftconv_c2r(sy, S * fo, n, m, 1.0 / (n * n), y.data_ptr(), sh), "fftconv_c2r")

    def region(fn, count):
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

    K = max(5, args.steps // 10)
    for i in range(max(2, args.warmup // 10)):
        step(i)
    wall, _ = region(step, K)
    log(f"[bench] fft: timed {K} layer steps: wall {wall * 1e3:.2f} ms")
    ops = {}
    for name, fn in (("fprop", op_f), ("bprop", op_b), ("accgrad", op_a)):
        _, ms = region(fn, K)
        ops[name] = round(ms / K, 4)
    stage_bytes = {"r2c_x": S * f * (n * n * 4 + P * 8), "r2c_w": fo * f * (k * k * 4 + P * 8),
                   "c2r_y": S * fo * (P * 8 + m * m * 4)}
    stages = {}
    for name, fn in (("r2c_x", st_r2c_x), ("r2c_w", st_r2c_w), ("cmul", st_cmul), ("c2r_y", st_c2r)):
        _, ms = region(fn, K)
        us = ms * 1e3 / K
        stages[name] = {"mean_us": round(us, 2)}
        if name in stage_bytes:
            stages[name]["bytes"] = stage_bytes[name]
            stages[name]["GBps"] = round(stage_bytes[name] / (us * 1e-6) / 1e9, 1)
    # Copy kernel over the input maps (read + write), same run: the HBM
    # ceiling at this size, and the calibration of the traffic counters.
    cbytes = S * f * n * n * 4
    csrc = torch.empty(cbytes, dtype=torch.uint8, device=dev)
    cdst = torch.empty(cbytes, dtype=torch.uint8, device=dev)

    def k_copy(_):
        _lib.check(lib.meswish_copy(csrc.data_ptr(), cdst.data_ptr(), cbytes, sh), "meswish_copy")

    for i in range(3):
        k_copy(i)
    _, cms = region(k_copy, K)
    copy_us = cms * 1e3 / K
    del csrc, cdst
    fft_traffic = fft_traffic_from_profile()
    cm_flops = 8 * S * fo * f * P
    cm_us = stages["cmul"]["mean_us"]
    cm_tf = cm_flops / (cm_us * 1e-6) / 1e12
    stages["cmul"].update({"flops": cm_flops, "TFLOPs": round(cm_tf, 2),
                           "bytes": P * 8 * (S * f + fo * f + S * fo)})

    # PyTorch's direct convolution (MIOpen) on the same layer: forward and
    # both gradients.
    tx = x.clone().requires_grad_(True)
    tw = w.clone().requires_grad_(True)

    def torch_step(_):
        ty = torch.nn.functional.conv2d(tx, tw)
        ty.backward(g)

    for i in range(3):
        torch_step(i)
    twall, _ = region(torch_step, K)
    direct_flops = 2 * S * fo * f * m * m * k * k   # per operation
    step_ms = wall * 1e3 / K

    result = {
        "metric": f"layer steps/s (fprop + bprop + accgrad), FFT convolution S={S} f={f} f'={fo} "
                  f"n={n} k={k} fp32, 1 MI355X",
        "value": round(1e3 / step_ms, 2),
        "unit": "layer steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": max(2, args.warmup // 10),
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"FFT convolution layer, minibatch {S}, {f} -> {fo} feature maps, "
                               f"{n}x{n} inputs, {k}x{k} kernels, fp32",
                   "S": S, "f": f, "fo": fo, "n": n, "k": k, "bins": P,
                   "frequency_buffer_bytes": fb},
        "ms_per_operation": ops,
        "stages_fprop": stages,
        "direct_equivalent_TFLOPs": round(3 * direct_flops / (step_ms * 1e-3) / 1e12, 2),
        "roofline": {"kernel": "cgemm_kernel (per-bin complex products on the matrix cores, forward)",
                     "bound": "mfma", "achieved": round(cm_tf, 2), "peak": PEAK_FP32_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(cm_tf / PEAK_FP32_MFMA_TFLOPS, 4),
                     "traffic": fft_traffic[0], "traffic_note": fft_traffic[1],
                     "bytes_per_launch": stages["cmul"]["bytes"],
                     "flops_per_launch": cm_flops, "mean_launch_us": cm_us,
                     "matrix_core_flops_per_launch": cm_flops * 3 // 4,
                     "matrix_core_frac": round(cm_tf * 0.75 / PEAK_FP32_MFMA_TFLOPS, 4),
                     "note": "achieved counts the product's 8 M N K flops per bin; the kernel "
                             "forms each complex term from three real matrix-core products "
                             "(Gauss), so the matrix cores execute three quarters of them"},
        "copy_ceiling": {"bytes": 2 * cbytes, "mean_us": round(copy_us, 2),
                         "GBps": round(2 * cbytes / (copy_us * 1e-6) / 1e9, 1)},
        "torch_direct_conv_same_layer": {"ms_per_step": round(twall * 1e3 / K, 4),
                                         "note": "F.conv2d forward + autograd input and weight "
                                                 "gradients (MIOpen), fp32"},
    }
    if not args.no_cpu_baseline:
        import numpy as np
        from oracle import fft_oracle
        # Runs over successive pairs of minibatch samples, each a layer step
        # on 2 of the S samples, until the time bound; scaled to all S.
        sub, pos = 2, [0]

        def run():
            lo = pos[0] % S
            pos[0] += sub
            fft_oracle.fprop_fft(L.x[lo:lo + sub], L.w)
            fft_oracle.bprop_fft(L.g[lo:lo + sub], L.w, n)
            fft_oracle.accgrad_fft(L.x[lo:lo + sub], L.g[lo:lo + sub], k)
        ct, runs, total = time_cpu(run, args)
        est_ms = ct * 1e3 * S / sub
        result["cpu_baseline"] = {"value": round(1e3 / est_ms, 4), "unit": "layer steps/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": f"{runs} runs over {sub} of the {S} minibatch samples "
                                            f"each, numpy binary64 spectral path, median "
                                            f"{ct:.2f} s per run ({total:.1f} s in all), "
                                            f"scaled by {S // sub}"}
        log(f"[bench] fft: cpu baseline {ct:.2f} s per {sub} samples x {runs}")
        del np
    return result


def measure_grouped(args, lib, torch, dev):
    """Config 5: the grouped launch (one kernel per direction) over the seven
    EfficientNet-shaped bf16 tensors, against seven single launches per
    direction, on SETS rotating copies."""
    from memory_efficient_activation_amd import _lib, inputs

    w = inputs.make(5)
    dt, alpha = _lib.BF16, float(w.alpha)

    def to_dev(a):
        return torch.from_numpy(a).view(torch.int16).view(torch.bfloat16).to(dev)

    sets = []
    for _ in range(SETS):
        xs = [to_dev(a) for a in w.xs]
        dys = [to_dev(a) for a in w.dys]
        ys = [torch.empty_like(x) for x in xs]
        dxs = [torch.empty_like(x) for x in xs]
        fd = (_lib.FwdDesc * len(xs))(*[_lib.FwdDesc(x.data_ptr(), y.data_ptr(), x.numel())
                                        for x, y in zip(xs, ys)])
        bd = (_lib.BwdDesc * len(xs))(*[_lib.BwdDesc(x.data_ptr(), d.data_ptr(), g.data_ptr(),
                                                     x.numel()) for x, d, g in zip(xs, dys, dxs)])
        sets.append(dict(xs=xs, dys=dys, ys=ys, dxs=dxs, fd=fd, bd=bd))
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    count = len(w.xs)
    total = sum(a.size for a in w.xs)
    fwd_b, bwd_b = 2 * 2 * total, 3 * 2 * total

    def g_fwd(j):
        _lib.check(lib.swish_fwd_grouped(sets[j % SETS]["fd"], count, alpha, dt, sh), "grouped")

    def g_bwd(j):
        _lib.check(lib.swish_bwd_grouped(sets[j % SETS]["bd"], count, alpha, dt, sh), "grouped")

    def s_fwd(j):
        for d in sets[j % SETS]["fd"]:
            _lib.check(lib.swish_fwd(d.x, d.y, d.n, alpha, dt, sh), "swish_fwd")

    def s_bwd(j):
        for d in sets[j % SETS]["bd"]:
            _lib.check(lib.swish_bwd(d.x, d.dy, d.dx, d.n, alpha, dt, sh), "swish_bwd")

    def region(fn, k):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        for i in range(k):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, a.elapsed_time(b)

    K = args.steps
    for i in range(args.warmup):
        g_fwd(2 * i)
        g_bwd(2 * i + 1)
    wall, _ = region(lambda i: (g_fwd(2 * i), g_bwd(2 * i + 1)), K)
    _, gb_ms = region(g_bwd, K)
    _, gf_ms = region(g_fwd, K)
    for i in range(3):
        s_fwd(2 * i)
        s_bwd(2 * i + 1)
    swall, _ = region(lambda i: (s_fwd(2 * i), s_bwd(2 * i + 1)), K)
    step_b = fwd_b + bwd_b
    value = step_b * K / wall / 1e9
    bwd_us = gb_ms * 1e3 / K
    bwd_gbps = bwd_b / (bwd_us * 1e-6) / 1e9
    result = {
        "metric": "HBM GB/s + fraction of peak, grouped Swish fwd+bwd over 7 EfficientNet "
                  "MBConv-shaped bf16 tensors (70M elements), 1 MI355X",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / K, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "io_dtype": "bf16", "data": "synthetic",
        "config": {"workload": "grouped Swish fwd+bwd, one launch per direction over 7 bf16 NHWC "
                               "tensors at batch 32 (112^2x96, 56^2x144, 28^2x240, 14^2x480, "
                               "14^2x672, 7^2x1152, 7^2x1280)",
                   "tensors": count, "elements": total, "bytes_per_step": step_b,
                   "buffer_sets": SETS},
        "frac_peak": round(value / PEAK_HBM_GBPS, 4),
        "fwd": {"bytes": fwd_b, "mean_us": round(gf_ms * 1e3 / K, 2),
                "GBps": round(fwd_b / (gf_ms * 1e-3 / K) / 1e9, 1)},
        "roofline": {"kernel": "act_group_kernel<bf16, bwd, swish> (grouped backward)",
                     "bound": "hbm", "achieved": round(bwd_gbps, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(bwd_gbps / PEAK_HBM_GBPS, 4), "traffic": None,
                     "traffic_note": "counters taken for the single-tensor kernels",
                     "bytes_per_launch": bwd_b, "mean_launch_us": round(bwd_us, 2)},
        "single_launches_same_step": {"launches_per_step": 2 * count,
                                      "ms_per_step": round(swall * 1e3 / K, 5),
                                      "GBps": round(step_b * K / swall / 1e9, 1)},
    }
    if not args.no_cpu_baseline:
        from oracle import Oracle
        orc = Oracle()
        threads = len(os.sched_getaffinity(0))
        def run():
            orc.fwd_grouped(w.xs, alpha, threads=threads)
            orc.bwd_grouped(w.xs, w.dys, alpha, threads=threads, want_scale=False)
        ct, runs, spent = time_cpu(run, args)
        result["cpu_baseline"] = {"value": round(step_b / ct / 1e9, 3), "unit": "GB/s",
                                  "cores": threads, "kind": "oracle",
                                  "sample": f"the full workload (7 tensors, {total} elements) "
                                            f"fwd+bwd, binary64 C oracle, median of {runs} runs "
                                            f"({ct:.2f} s each, {spent:.1f} s in all)"}
    return result


# Stationary point of Swish' in t = alpha x: 1 + t (1 - sigma(t)) = 0 at
# t0 = -(1 + W(1/e)); results near it cancel (their error is judged against
# the size of the terms).
T0_SWISH_GRAD = -1.2784645427610738
SCRUB_BYTES = 1 << 30   # 4x the 256 MB Infinity Cache


def _pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]


def measure_report(args, lib, torch, dev, cfgs):
    """The per-launch protocol, one JSON line per workload and direction.

    For each direction: W warm launches, then R launches timed one by one
    with a HIP event pair each on the launch stream, every one preceded
    (outside its pair) by a read of a 1 GiB buffer that evicts the caches;
    the median and p10/p90 of those times give GB/s.  Also: the same R
    launches back to back without the fill ("hot"), the 16-byte copy kernel
    over one tensor under the same protocol (the practical ceiling), the
    GPU results against the oracle (largest error under the parity rule,
    elements beyond it), the counts of the two hazard bands (subnormal
    outputs; |alpha x - t0| < 0.05 in the backward), and the oracle's time
    on the host: all threads (median of 3) and one thread (on the first
    2^22 elements, scaled)."""
    import numpy as np
    from memory_efficient_activation_amd import _lib, accounting, inputs
    import oracle
    from oracle.compare import bf16_report, f32_report

    orc = oracle.Oracle()
    threads = len(os.sched_getaffinity(0))
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    scrub = torch.zeros(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)

    def to_dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(dev)

    def to_host(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    def timed(fn, reps, scrubbed):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in evs:
            if scrubbed:
                # Read, not write: a read pass leaves the caches holding
                # clean lines, so the timed kernel pays no write-back of
                # the scrub's own data (a fill of the buffer left up to
                # 256 MB of dirty lines, written back inside the timed pair).
                scrub.sum()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in evs]   # microseconds

    out = []
    for c in cfgs:
        w = inputs.make(c)
        dt = _lib.BF16 if w.dtype == "bf16" else _lib.F32
        esize = 2 if w.dtype == "bf16" else 4
        n, alpha = w.numel, float(w.alpha)
        reps = args.report_reps * (10 if c == 1 else 1)
        xs = [to_dev(a) for a in w.xs]
        dys = [to_dev(a) for a in w.dys]
        ys = [torch.empty_like(x) for x in xs]
        dxs = [torch.empty_like(x) for x in xs]
        if c == 5:
            fd = (_lib.FwdDesc * len(xs))(*[_lib.FwdDesc(x.data_ptr(), y.data_ptr(), x.numel())
                                            for x, y in zip(xs, ys)])
            bd = (_lib.BwdDesc * len(xs))(*[_lib.BwdDesc(x.data_ptr(), d.data_ptr(), g.data_ptr(),
                                                         x.numel()) for x, d, g in zip(xs, dys, dxs)])

            def fwd():
                _lib.check(lib.swish_fwd_grouped(fd, len(xs), alpha, dt, sh), "swish_fwd_grouped")

            def bwd():
                _lib.check(lib.swish_bwd_grouped(bd, len(xs), alpha, dt, sh), "swish_bwd_grouped")
        else:
            x, dy, y, dx = xs[0], dys[0], ys[0], dxs[0]

            def fwd():
                _lib.check(lib.swish_fwd(x.data_ptr(), y.data_ptr(), n, alpha, dt, sh), "swish_fwd")

            def bwd():
                _lib.check(lib.swish_bwd(x.data_ptr(), dy.data_ptr(), dx.data_ptr(), n, alpha, dt, sh),
                           "swish_bwd")
        csrc = torch.empty(n * esize, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)

        def copy():
            _lib.check(lib.meswish_copy(csrc.data_ptr(), cdst.data_ptr(), n * esize, sh), "meswish_copy")

        for _ in range(5):
            fwd()
            bwd()
            copy()
        t_copy = timed(copy, reps, True)
        copy_med = statistics.median(t_copy)
        copy_gbps = 2 * n * esize / (copy_med * 1e-6) / 1e9
        # The oracle on the same inputs: values for the errors, and times.
        x64 = np.concatenate([inputs.decode(a).astype(np.float64) for a in w.xs])
        for direction, fn in (("fwd", fwd), ("bwd", bwd)):
            t_s = timed(fn, reps, True)
            t_h = timed(fn, reps, False)
            nbytes = (accounting.fwd_bytes(n, w.dtype) if direction == "fwd"
                      else accounting.bwd_bytes(n, w.dtype))
            med = statistics.median(t_s)
            got = np.concatenate([to_host(t).ravel() for t in (ys if direction == "fwd" else dxs)])

            def run_oracle(th, k=None):
                if direction == "fwd":
                    return [orc.fwd(a[:k], alpha, threads=th) for a in w.xs]
                return [orc.bwd(a[:k], d[:k], alpha, threads=th, want_scale=k is None)
                        for a, d in zip(w.xs, w.dys)]

            cpu_t = []
            for _ in range(3):
                c0 = time.perf_counter()
                res = run_oracle(threads)
                cpu_t.append(time.perf_counter() - c0)
            k1 = 1 << 22
            done = sum(min(a.size, k1) for a in w.xs)
            c0 = time.perf_counter()
            run_oracle(1, k1)
            t1 = (time.perf_counter() - c0) * n / done
            if direction == "fwd":
                want = np.concatenate([r.ravel() for r in res])
                scale = None
            else:
                want = np.concatenate([r[0].ravel() for r in res])
                scale = np.concatenate([r[1].ravel() for r in res])
            rep = (bf16_report(got, want) if w.dtype == "bf16" else f32_report(got, want, scale))
            wv = inputs.decode(want).astype(np.float64)
            bands = {"subnormal_outputs": int(np.count_nonzero((wv != 0) & (np.abs(wv) < 2.0 ** -126)))}
            if direction == "bwd":
                bands["near_t0"] = int(np.count_nonzero(np.abs(alpha * x64 - T0_SWISH_GRAD) < 0.05))
            cpu_med = statistics.median(cpu_t)
            line = {
                "report": "per-launch protocol", "config_index": c, "direction": direction,
                "workload": w.name, "io_dtype": w.dtype, "n": n, "bytes": nbytes, "reps": reps,
                "t_median_us": round(med, 2), "t_p10_us": round(_pct(t_s, 0.1), 2),
                "t_p90_us": round(_pct(t_s, 0.9), 2),
                "GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
                "frac_peak": round(nbytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                "hot": {"t_median_us": round(statistics.median(t_h), 2),
                        "GBps": round(nbytes / (statistics.median(t_h) * 1e-6) / 1e9, 1),
                        "note": "back to back, no cache scrub"},
                "copy": {"bytes": 2 * n * esize, "t_median_us": round(copy_med, 2),
                         "GBps": round(copy_gbps, 1)},
                "frac_copy": round(nbytes / (med * 1e-6) / 1e9 / copy_gbps, 4),
                "elems_per_s": round(n / (med * 1e-6), 1),
                "retained_bytes": {"memory_efficient": accounting.retained_bytes(n, w.dtype),
                                   "naive_3_maps": accounting.retained_bytes(n, w.dtype, naive=True)},
                "max_err": ({"max_ulp": rep["max_ulp"], "n_off_by_one": rep["n_off_by_one"]}
                            if w.dtype == "bf16" else {"max_rel": rep["max_rel"]}),
                "n_bad": rep["n_bad"], "parity_ok": rep["ok"],
                "bands": bands,
                "cpu": {"cores": threads, "t_s": round(cpu_med, 4),
                        "GBps": round(nbytes / cpu_med / 1e9, 3),
                        "t_1thread_s": round(t1, 3), "GBps_1thread": round(nbytes / t1 / 1e9, 3),
                        "kind": "oracle"},
                "gpu_over_cpu": round(cpu_med / (med * 1e-6), 1),
            }
            log(f"[report] config {c} {direction}: {line['t_median_us']} us, {line['GBps']} GB/s, "
                f"parity {rep['ok']}")
            out.append(line)
        del xs, dys, ys, dxs, csrc, cdst
        torch.cuda.empty_cache()
    return out


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the Swish path is element-wise and shards "
              "with no communication (each GPU runs on its local tensor), so the one-GPU "
              "figure times N is the N-GPU figure. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from memory_efficient_activation_amd import _lib, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a HIP GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = _lib.library()
    if args.dense:
        print(json.dumps(measure_dense(args, lib, torch, dev)), flush=True)
        return
    if args.fft:
        print(json.dumps(measure_fft(args, lib, torch, dev)), flush=True)
        return
    if args.report:
        cfgs = [args.config] if "--config" in sys.argv else [1, 2, 3, 4, 5]
        for line in measure_report(args, lib, torch, dev, cfgs):
            print(json.dumps(line), flush=True)
        return
    if args.grouped or args.config == 5:
        print(json.dumps(measure_grouped(args, lib, torch, dev)), flush=True)
        return
    if args.act != "swish" and args.config != 3:
        print("--act measures the bf16 [8,2048,4096] workload (--config 3)", file=sys.stderr)
        sys.exit(2)

    t_gen = time.perf_counter()
    w = inputs.make(args.config)
    log(f"[bench] inputs generated in {time.perf_counter() - t_gen:.1f} s: {w.name}, n={w.numel}")
    rig = Rig(torch, w, dev)
    acts = FAMILY if args.act == "all" else [args.act]
    for act in acts:
        print(json.dumps(measure(args, act, rig, w, lib, torch)), flush=True)


if __name__ == "__main__":
    main()
