"""Summarise rocprofv3 CSV output of bench.py into short markdown tables.

Usage (after the rocprofv3 runs listed in each summary's header):

    python -m memory_efficient_activation_amd.rocprof_summary trace DIR [--io f32]
    python -m memory_efficient_activation_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR [--io f32]
    python -m memory_efficient_activation_amd.rocprof_summary timeline DIR [WINDOW] [--io f32]
    python -m memory_efficient_activation_amd.rocprof_summary valu DIR [--io f32] [--elements N]
    python -m memory_efficient_activation_amd.rocprof_summary rare [WORKLOAD]
    python -m memory_efficient_activation_amd.rocprof_summary grouped-trace DIR [STEPS]
    python -m memory_efficient_activation_amd.rocprof_summary dense-trace DIR f32|bf16
    python -m memory_efficient_activation_amd.rocprof_summary dense-traffic FETCH_DIR WRITE_DIR f32|bf16
    python -m memory_efficient_activation_amd.rocprof_summary fft-trace DIR
    python -m memory_efficient_activation_amd.rocprof_summary fft-traffic FETCH_DIR WRITE_DIR
    python -m memory_efficient_activation_amd.rocprof_summary counters DIR act|dense|fft [--io f32]

``trace``   reads ``*_kernel_stats.csv`` and ``*_kernel_trace.csv`` from a
            ``--kernel-trace --stats --output-format csv`` run and prints the
            per-kernel averages, plus the per-region averages of bench.py's
            three timed regions (alternating steps, backward only, forward
            only).
``traffic`` reads ``*_counter_collection.csv`` of one ``--pmc FETCH_SIZE``
            run and one ``--pmc WRITE_SIZE`` run, calibrates each counter on
            the plain copy kernel (which reads and writes exactly
            ``bytes`` = 2 b n per launch), and prints the HBM bytes per
            launch of the forward and backward kernels next to their
            algorithmic bytes, with the sha256 of the kernel source.
``timeline`` the kernel times of a ``trace`` run (or of a ``--pmc
            GRBM_GUI_ACTIVE`` run, then with the counter's cycles per
            microsecond) in windows of consecutive launches, in run order.
``valu``    vector-ALU counters of ``bench.py --act all`` per kernel: VALUBusy
            and vector instructions per element.
``grouped-trace`` the kernel times of ``bench.py --grouped``: the grouped
            kernels in the timed steps and back to back, and the step as
            fourteen single launches.
``dense-*`` the same for ``bench.py --dense`` (DenseNet-BC-100 block 1,
            layer 16: 204 channels of 64 x 32 x 32; its newest source has 12):
            forward 2 C M b bytes per launch, backward reduction 2 C M b,
            backward apply 3 C M b, statistics 12 M b, copy 2 C M b.
``fft-*``   the same for ``bench.py --fft`` (S=128, f=96, f'=256, n=32, k=7):
            each launch is attributed to its stage by kernel and grid size;
            transforms count their real maps and half spectra (8 bytes per
            bin), products their three spectrum arrays and 8 M N K P flops.
``counters`` every counter of one ``--pmc`` run, as the mean per dispatch
            of each kernel (grouped as the family's other modes group them),
            with the sha256 of the family's kernel sources.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("meswish.hip", "act_math.h")]

N = 8 * 2048 * 4096          # elements of the benchmark tensor
# I/O type of the summarised run (the element type of act_vec_kernel's
# first template argument): "bf16" (the headline workload) or "f32" (the
# binary32 workload of the same shape); set_io() switches.
IO = "bf16"
IO_TYPE = {"bf16": "meswish::bf16_t", "f32": "float"}
ESIZE = {"bf16": 2, "f32": 4}
COPY_BYTES = ESIZE[IO] * N   # bytes the copy kernel reads (and writes) per launch
ALGO = {"fwd": 2 * COPY_BYTES, "bwd": 3 * COPY_BYTES, "copy": 2 * COPY_BYTES}


def set_io(io: str, elements: int | None = None) -> None:
    """Summarise runs of I/O type `io` over tensors of `elements` elements
    (default the [8, 2048, 4096] tensor)."""
    global IO, N, COPY_BYTES, ALGO
    if io not in ESIZE:
        raise SystemExit(f"unknown I/O type {io!r} (bf16 or f32)")
    IO = io
    if elements is not None:
        N = int(elements)
    COPY_BYTES = ESIZE[io] * N
    ALGO = {"fwd": 2 * COPY_BYTES, "bwd": 3 * COPY_BYTES, "copy": 2 * COPY_BYTES}


# Activation codes of act_vec_kernel's third template argument; 8 is Swish
# with alpha exactly 1 (the library's shorter backward).
ACT_NAMES = {0: "swish", 1: "relu", 2: "leaky_relu", 3: "sigmoid", 4: "tanh", 5: "gelu",
             6: "gelu_tanh", 8: "swish"}


def _vec_re() -> str:
    return r"act_vec_kernel<" + re.escape(IO_TYPE[IO]) + r", (true|false), (\d+)>"


def kind(name: str, act: str = "swish") -> str:
    """'fwd' / 'bwd' for the vector kernel (of the current I/O type) of
    activation `act`, 'copy' for the copy kernel, 'other' otherwise."""
    m = re.search(_vec_re(), name)
    if m:
        if ACT_NAMES.get(int(m.group(2))) != act:
            return "other"
        return "bwd" if m.group(1) == "true" else "fwd"
    if "copy16_kernel" in name:
        return "copy"
    return "other"


def act_of(name: str) -> str:
    m = re.search(_vec_re(), name)
    return ACT_NAMES.get(int(m.group(2)), "") if m else ""


def _one(pattern: str) -> str:
    hits = glob.glob(pattern)
    if len(hits) != 1:
        raise SystemExit(f"expected one file matching {pattern}, found {hits}")
    return hits[0]


def trace(d: str) -> str:
    stats = list(csv.DictReader(open(_one(os.path.join(d, "*_kernel_stats.csv")))))
    rows = list(csv.DictReader(open(_one(os.path.join(d, "*_kernel_trace.csv")))))
    out = ["| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in stats:
        out.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    seq = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                  kind(r["Kernel_Name"], act_of(r["Kernel_Name"]) or "swish"),
                  act_of(r["Kernel_Name"])) for r in rows)
    seq = [(s_, e_, (f"{a}:{k}" if a and k in ("fwd", "bwd") else k)) for s_, e_, k, a in seq]
    runs, cur = [], None
    for i, (_, _, k) in enumerate(seq):
        if cur and cur[0] == k:
            cur[2] = i
        else:
            if cur:
                runs.append(cur)
            cur = [k, i, i]
    if cur:
        runs.append(cur)
    out += ["", "| region (consecutive launches) | launches | mean kernel time (us) | "
                "algorithmic GB/s |", "|---|---|---|---|"]
    alt = [r for r in seq if r[2] in ("swish:fwd", "swish:bwd")]
    # The alternating region is the longest run of fwd/bwd pairs.
    best, start = (0, 0), None
    for i in range(len(alt)):
        if i and alt[i][2] != alt[i - 1][2]:
            start = i - 1 if start is None else start
            if i - start + 1 > best[0]:
                best = (i - start + 1, start)
        else:
            start = None
    if best[0] > 4:
        seg = alt[best[1]:best[1] + best[0]]
        for k in ("swish:fwd", "swish:bwd"):
            d_ = [e - s for s, e, kk in seg if kk == k]
            t = statistics.fmean(d_)
            out.append(f"| alternating swish fwd/bwd steps: {k.split(':')[1]} | {len(d_)} | "
                       f"{t / 1e3:.2f} | {ALGO[k.split(':')[1]] / t:.0f} |")
    for k, a, b in runs:
        base = k.split(":")[-1]
        if b - a >= 4 and base in ALGO:
            d_ = [seq[i][1] - seq[i][0] for i in range(a, b + 1)]
            t = statistics.fmean(d_)
            out.append(f"| {k} only, back to back | {len(d_)} | {t / 1e3:.2f} | "
                       f"{ALGO[base] / t:.0f} |")
    return "\n".join(out)


def timeline(d: str, window: int = 10) -> str:
    """Kernel times through the run, in windows of `window` launches of one
    kind: whether a kernel keeps its speed over a long stretch of launches.
    With a directory of a ``--pmc GRBM_GUI_ACTIVE`` run instead of a kernel
    trace, each window also gives the counter's cycles per microsecond of
    kernel time."""
    trace_csv = glob.glob(os.path.join(d, "*_kernel_trace.csv"))
    cycles = {}
    if trace_csv:
        rows = list(csv.DictReader(open(_one(os.path.join(d, "*_kernel_trace.csv")))))
    else:
        rows = [r for r in csv.DictReader(open(_one(os.path.join(d, "*_counter_collection.csv"))))
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE"]
        cycles = {r["Dispatch_Id"]: float(r["Counter_Value"]) for r in rows}
    seq = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r.get("Dispatch_Id", ""),
                  kind(r["Kernel_Name"], act_of(r["Kernel_Name"]) or "swish"),
                  act_of(r["Kernel_Name"])) for r in rows)
    seq = [x for x in seq if x[3] in ALGO]
    if not seq:
        return "(no activation or copy kernels)"
    t0 = seq[0][0]

    def region(i):
        # "fwd/bwd" inside the alternating steps (a neighbour of the other
        # kind and, one further, one of the same), else the launch's own kind.
        act, k = seq[i][4], seq[i][3]

        def at(j):
            return seq[j][3] if 0 <= j < len(seq) and seq[j][4] == act else None
        for d_ in (-1, 1):
            if k != "copy" and at(i + d_) not in (None, k) and at(i + 2 * d_) == k:
                return "fwd/bwd"
        return k
    regions = [region(i) for i in range(len(seq))]
    head = "| window | launches | starts at (ms) | fwd (us) | bwd (us) | copy (us) | GB/s |"
    if cycles:
        head += " cycles per us |"
    out = [head, "|" + "---|" * (head.count("|") - 1)]
    i = 0
    while i < len(seq):
        a, reg = seq[i][4] or "copy", regions[i]
        j = i
        # A window: up to `window` consecutive launches (steps, when
        # alternating) of one activation in one region of the run.
        limit = 2 * window if reg == "fwd/bwd" else window
        while (j < len(seq) and (seq[j][4] or "copy") == a and regions[j] == reg
               and j - i < limit):
            j += 1
        w = seq[i:j]
        mean = {}
        for k in ("fwd", "bwd", "copy"):
            d_ = [e - s for s, e, _, kk, _ in w if kk == k]
            mean[k] = statistics.fmean(d_) / 1e3 if d_ else None
        tot_b = sum(ALGO[kk] for _, _, _, kk, _ in w)
        tot_t = sum(e - s for s, e, _, _, _ in w)
        cells = [f"{a} {reg}" if a != "copy" else a, f"{len(w)}", f"{(w[0][0] - t0) / 1e6:.2f}"]
        cells += [f"{mean[k]:.1f}" if mean[k] is not None else "" for k in ("fwd", "bwd", "copy")]
        cells.append(f"{tot_b / tot_t:.0f}")
        if cycles:
            cyc = sum(cycles.get(x[2], 0.0) for x in w)
            cells.append(f"{cyc / (tot_t / 1e3):.0f}")
        out.append("| " + " | ".join(cells) + " |")
        i = j
    return "\n".join(out)


GROUPED_ELEMS = 70_045_696   # the seven EfficientNet-shaped tensors of the grouped bench


def grouped_trace(d: str, steps: int = 200) -> str:
    """``bench.py --grouped``: the grouped kernels in the timed alternating
    steps (the last `steps` of them), back to back, and the same step as
    fourteen single launches."""
    stats = list(csv.DictReader(open(_one(os.path.join(d, "*_kernel_stats.csv")))))
    rows = list(csv.DictReader(open(_one(os.path.join(d, "*_kernel_trace.csv")))))
    out = ["| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in stats:
        out.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")

    def lab(name):
        m = re.search(r"act_(group|vec)_kernel<meswish::bf16_t, (true|false), [08]>", name)
        if not m:
            return None
        return ("g" if m.group(1) == "group" else "s") + ("b" if m.group(2) == "true" else "f")
    seq = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), lab(r["Kernel_Name"]))
                 for r in rows)
    seq = [x for x in seq if x[2]]
    kinds = [k for _, _, k in seq]
    fb = {"f": 4 * GROUPED_ELEMS, "b": 6 * GROUPED_ELEMS}
    out += ["", "| region | launches | mean kernel time (us) | algorithmic GB/s |",
            "|---|---|---|---|"]
    # Alternating grouped steps: the longest run of gf/gb pairs; its last
    # `steps` steps are the timed ones.
    best, i = (0, 0), 0
    while i < len(kinds):
        j = i
        while j < len(kinds) and kinds[j] == ("gf" if (j - i) % 2 == 0 else "gb"):
            j += 1
        if j - i > best[1] - best[0]:
            best = (i, j)
        i = max(j, i + 1)
    seg = seq[max(best[0], best[1] - 2 * steps):best[1]]
    for k in ("gf", "gb"):
        d_ = [e - s_ for s_, e, kk in seg if kk == k]
        t = statistics.fmean(d_)
        out.append(f"| grouped {'forward' if k == 'gf' else 'backward'}, timed alternating steps "
                   f"| {len(d_)} | {t / 1e3:.2f} | {fb[k[1]] / t:.0f} |")
    for k, name in (("gb", "grouped backward only, back to back"),
                    ("gf", "grouped forward only, back to back")):
        runs, cur = [], []
        for x in seq[best[1]:]:
            if x[2] == k:
                cur.append(x)
            elif cur:
                runs.append(cur)
                cur = []
        if cur:
            runs.append(cur)
        r_ = max(runs, key=len)
        t = statistics.fmean(e - s_ for s_, e, _ in r_)
        out.append(f"| {name} | {len(r_)} | {t / 1e3:.2f} | {fb[k[1]] / t:.0f} |")
    single = [x for x in seq if x[2] in ("sf", "sb")]
    if single:
        n_steps = len(single) // 14
        t = sum(e - s_ for s_, e, _ in single) / max(n_steps, 1)
        out.append(f"| single launches, 14 per step (kernel time per step) | {len(single)} | "
                   f"{t / 1e3:.2f} | {(fb['f'] + fb['b']) / t:.0f} |")
    return "\n".join(out)


def valu(d: str) -> str:
    """A ``--pmc VALUBusy SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_WAVES`` run
    of ``bench.py --act all``: per kernel, the mean kernel time, VALUBusy
    (rocprofv3's derived metric: percent of GPU time the vector ALUs are
    issuing) and vector instructions per element (per-lane instructions:
    SQ_INSTS_VALU counts wavefront instructions of 64 lanes)."""
    rows = list(csv.DictReader(open(_one(os.path.join(d, "*_counter_collection.csv")))))
    agg = {}
    for r in rows:
        name = r["Kernel_Name"]
        k = kind(name, act_of(name) or "swish")
        if k not in ALGO:
            continue
        key = (act_of(name) or "copy", k)
        x = agg.setdefault(key, {}).setdefault(r["Dispatch_Id"], {
            "dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
        x[r["Counter_Name"]] = float(r["Counter_Value"])
    out = ["| kernel | launches | mean time (us) | VALUBusy (%) | vector instructions per "
           "element | of which transcendental |", "|---|---|---|---|---|---|"]
    for (a, k), v in agg.items():
        ds = list(v.values())

        def mean(c):
            return statistics.fmean(x[c] for x in ds)
        label = "copy" if a == "copy" else f"{a} {k}"
        out.append(f"| {label} | {len(ds)} | {mean('dur'):.1f} | {mean('VALUBusy'):.1f} | "
                   f"{mean('SQ_INSTS_VALU') * 64 / N:.2f} | "
                   f"{mean('SQ_INSTS_VALU_TRANS_F32') * 64 / N:.2f} |")
    return "\n".join(out)


def rare_rate(index: int = 4) -> str:
    """How often the binary32 Swish kernels enter their rare branch on
    workload `index` (default 4: alpha 1.5, 1 % of x in +-[20, 90]): an
    element is rare where |fl(x c_hi)| > 125 (c_hi = fl(-alpha log2 e)); a
    wave of the binary32 kernels covers 64 lanes x 4 consecutive elements
    and takes the branch if any of them is rare, then runs one masked
    region per element slot j = 0..3 that some lane needs.  Computed from
    the workload's own inputs, exactly."""
    import numpy as np

    from . import inputs
    w = inputs.make(index)
    x = inputs.decode(w.xs[0]).astype(np.float32)
    c_hi = np.float32(-float(np.float32(w.alpha)) * 1.4426950408889634)
    v = (x * c_hi).astype(np.float32)
    rare = np.abs(v) > np.float32(125.0)
    per = 256  # elements per wave: 64 lanes x one 16-byte vector of 4
    n = x.size - x.size % per
    waves = rare[:n].reshape(-1, 64, 4)
    any_wave = waves.any(axis=(1, 2))
    slots = waves.any(axis=1)          # [wave, j]: some lane's element j is rare
    out = [f"workload {index}: {w.name}, {x.size} elements, alpha {w.alpha}",
           f"rare elements: {int(rare.sum())} ({rare.mean() * 100:.3f} %)",
           f"waves (256 elements) entering the rare branch: {int(any_wave.sum())} of "
           f"{any_wave.size} ({any_wave.mean() * 100:.1f} %)",
           f"masked regions run per wave (element slots needed, mean over all waves): "
           f"{slots.sum(axis=1).mean():.3f}",
           f"rare elements per entering wave (mean): {waves.sum(axis=(1, 2))[any_wave].mean():.2f}"]
    return "\n".join(out)


def _counter(d: str, name: str) -> dict:
    rows = list(csv.DictReader(open(_one(os.path.join(d, "*_counter_collection.csv")))))
    acc: dict = {}
    for r in rows:
        if r["Counter_Name"] == name:
            acc.setdefault(kind(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: statistics.fmean(v) for k, v in acc.items()}


def traffic(fetch_dir: str, write_dir: str) -> str:
    f = _counter(fetch_dir, "FETCH_SIZE")
    w = _counter(write_dir, "WRITE_SIZE")
    kib = COPY_BYTES / 1024
    cf, cw = kib / f["copy"], kib / w["copy"]
    h = hashlib.sha256()
    for path in SOURCES:
        h.update(open(path, "rb").read())
    sha = h.hexdigest()
    out = [f"calibration (copy kernel, {COPY_BYTES} B read and written per launch): "
           f"FETCH_SIZE reads {f['copy']:.1f} KiB -> factor {cf:.5f}; "
           f"WRITE_SIZE reads {w['copy']:.1f} KiB -> factor {cw:.5f}", "",
           "| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes (calibrated) | "
           "algorithmic bytes | ratio |", "|---|---|---|---|---|---|"]
    per = {}
    for k in ("fwd", "bwd", "copy"):
        b = (f[k] * cf + w[k] * cw) * 1024
        per[k] = b
        out.append(f"| {k} | {f[k]:.1f} | {w[k]:.1f} | {b:.0f} | {ALGO[k]} | {b / ALGO[k]:.5f} |")
    out += ["", f"traffic_bytes_per_launch: {per['bwd']:.0f}", f"kernel_source_sha256: {sha}"]
    return "\n".join(out)


DENSE_SOURCES = [os.path.join(HERE, "csrc", "dense_bn.hip")]
DENSE_C, DENSE_M, DENSE_NEW = 204, 64 * 32 * 32, 12


def dense_kind(name: str) -> str:
    for key, k in (("dense_bn::fwd_kernel", "fwd"), ("bwd_reduce_kernel", "reduce"),
                   ("bwd_apply_kernel", "apply"), ("stats_partial_kernel", "stats_partial"),
                   ("stats_final_kernel", "stats_final"), ("copy16_kernel", "copy")):
        if key in name:
            return k
    return "other"


def dense_algo(dtype: str) -> dict:
    b = 4 if dtype == "f32" else 2
    cmb = DENSE_C * DENSE_M * b
    return {"fwd": 2 * cmb, "reduce": 2 * cmb, "apply": 3 * cmb,
            "stats_partial": DENSE_NEW * DENSE_M * b, "copy": 2 * cmb}


def dense_trace(d: str, dtype: str) -> str:
    algo = dense_algo(dtype)
    stats = list(csv.DictReader(open(_one(os.path.join(d, "*_kernel_stats.csv")))))
    rows = list(csv.DictReader(open(_one(os.path.join(d, "*_kernel_trace.csv")))))
    out = ["| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in stats:
        out.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    acc: dict = {}
    for r in rows:
        k = dense_kind(r["Kernel_Name"])
        acc.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out += ["", "| kernel | launches | mean (us) | algorithmic bytes | algorithmic GB/s |",
            "|---|---|---|---|---|"]
    for k in ("fwd", "reduce", "apply", "stats_partial", "copy"):
        if k in acc:
            t = statistics.fmean(acc[k])
            out.append(f"| {k} | {len(acc[k])} | {t / 1e3:.2f} | {algo[k]} | {algo[k] / t:.0f} |")
    return "\n".join(out)


def dense_traffic(fetch_dir: str, write_dir: str, dtype: str) -> str:
    algo = dense_algo(dtype)

    def counter(d, name):
        rows = list(csv.DictReader(open(_one(os.path.join(d, "*_counter_collection.csv")))))
        acc: dict = {}
        for r in rows:
            if r["Counter_Name"] == name:
                acc.setdefault(dense_kind(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return {k: statistics.fmean(v) for k, v in acc.items()}

    f, w = counter(fetch_dir, "FETCH_SIZE"), counter(write_dir, "WRITE_SIZE")
    kib = algo["copy"] / 2 / 1024
    cf, cw = kib / f["copy"], kib / w["copy"]
    h = hashlib.sha256()
    for path in DENSE_SOURCES:
        h.update(open(path, "rb").read())
    out = [f"calibration (copy kernel, {algo['copy'] // 2} B read and written per launch): "
           f"FETCH_SIZE reads {f['copy']:.1f} KiB -> factor {cf:.5f}; "
           f"WRITE_SIZE reads {w['copy']:.1f} KiB -> factor {cw:.5f}", "",
           "| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes (calibrated) | "
           "algorithmic bytes | ratio |", "|---|---|---|---|---|---|"]
    per = {}
    for k in ("fwd", "reduce", "apply", "stats_partial", "copy"):
        if k in f and k in w:
            b = (f[k] * cf + w[k] * cw) * 1024
            per[k] = b
            out.append(f"| {k} | {f[k]:.1f} | {w[k]:.1f} | {b:.0f} | {algo[k]} | "
                       f"{b / algo[k]:.5f} |")
    out += ["", f"traffic_bytes_per_launch: {per['fwd']:.0f}",
            f"kernel_source_sha256: {h.hexdigest()}"]
    return "\n".join(out)


FFT = {"S": 128, "f": 96, "fo": 256, "n": 32, "k": 7}
FFT_SOURCES = [os.path.join(HERE, "csrc", "fft_conv.hip")]


def fft_stages():
    """(kernel key, maps) -> (stage, algorithmic bytes, flops) for the bench layer."""
    S, f, fo, n, k = FFT["S"], FFT["f"], FFT["fo"], FFT["n"], FFT["k"]
    m, P = n - k + 1, n * (n // 2 + 1)
    st = {}
    for name, B, mm in (("r2c x", S * f, n), ("r2c w", fo * f, k), ("r2c g", S * fo, m)):
        st[("r2c", B)] = (name, B * mm * mm * 4 + B * P * 8, 0)
    # The layer operations transform both inputs in one launch.
    for name, parts in (("r2c x+w (forward)", ((S * f, n), (fo * f, k))),
                        ("r2c g+w (input gradient)", ((S * fo, m), (fo * f, k))),
                        ("r2c g+x (weight gradient)", ((S * fo, m), (S * f, n)))):
        B = sum(b for b, _ in parts)
        st[("r2c", B)] = (name, sum(b * mm * mm * 4 + b * P * 8 for b, mm in parts), 0)
    for name, B, mm in (("c2r y (forward)", S * fo, m), ("c2r gx (input gradient)", S * f, n),
                        ("c2r gw (weight gradient)", fo * f, k)):
        st[("c2r", B)] = (name, B * P * 8 + B * mm * mm * 4, 0)
    flops = 8 * S * f * fo * P
    st[("cmul", 0)] = ("products, forward", P * 8 * (S * f + fo * f + S * fo), flops)
    st[("cmul", 1)] = ("products, input gradient", P * 8 * (S * fo + fo * f + S * f), flops)
    st[("cmul", 2)] = ("products, weight gradient", P * 8 * (S * fo + S * f + fo * f), flops)
    return st


def fft_key(r: dict):
    name = r["Kernel_Name"]
    if "copy16_kernel" in name:
        return ("copy", 0)
    maps_per_block = {8: 64, 16: 64, 32: 32, 64: 8}
    for kind in ("r2c", "c2r"):
        mm = re.search(kind + r"_kernel<(\d+)(?:, (?:true|false))?>", name)
        if mm:
            # Kernel traces give Grid_Size_X / Workgroup_Size_X, counter
            # collections Grid_Size / Workgroup_Size (1-D grids here).
            grid = int(r.get("Grid_Size_X") or r["Grid_Size"])
            blocks = grid // int(r.get("Workgroup_Size_X") or r["Workgroup_Size"])
            B = blocks * maps_per_block[int(mm.group(1))]
            # The last block may be partial: match the stage whose map count rounds up to B.
            for key in fft_stages():
                if key[0] == kind and -(-key[1] // maps_per_block[int(mm.group(1))]) == blocks:
                    return key
            return (kind, B)
    mm = re.search(r"cgemm(?:_mfma|_planar)?_kernel<(true|false), (true|false), (true|false), (true|false)(?:, \d+)*>", name)
    if mm:
        flags = tuple(x == "true" for x in mm.groups())
        return ("cmul", {(True, True, False, True): 0, (True, False, False, False): 1,
                         (False, False, True, False): 2}.get(flags, -1))
    return ("other", 0)


def fft_trace(d: str) -> str:
    st = fft_stages()
    stats = list(csv.DictReader(open(_one(os.path.join(d, "*_kernel_stats.csv")))))
    rows = list(csv.DictReader(open(_one(os.path.join(d, "*_kernel_trace.csv")))))
    out = ["| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in stats:
        out.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    acc: dict = {}
    for r in rows:
        key = fft_key(r)
        if key in st:
            acc.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out += ["", "| stage | launches | mean (us) | algorithmic bytes | GB/s | TFLOP/s |",
            "|---|---|---|---|---|---|"]
    for key, (name, nb, fl) in st.items():
        if key in acc:
            t = statistics.fmean(acc[key])
            tf = f"{fl / t / 1e3:.1f}" if fl else "-"
            out.append(f"| {name} | {len(acc[key])} | {t / 1e3:.2f} | {nb} | {nb / t:.0f} | {tf} |")
    return "\n".join(out)


def fft_traffic(fetch_dir: str, write_dir: str) -> str:
    st = fft_stages()

    def counter(d, cname):
        rows = list(csv.DictReader(open(_one(os.path.join(d, "*_counter_collection.csv")))))
        acc: dict = {}
        for r in rows:
            if r["Counter_Name"] == cname:
                acc.setdefault(fft_key(r), []).append(float(r["Counter_Value"]))
        return {k: statistics.fmean(v) for k, v in acc.items()}

    f, w = counter(fetch_dir, "FETCH_SIZE"), counter(write_dir, "WRITE_SIZE")
    cbytes = FFT["S"] * FFT["f"] * FFT["n"] ** 2 * 4
    cf, cw = cbytes / 1024 / f[("copy", 0)], cbytes / 1024 / w[("copy", 0)]
    h = hashlib.sha256()
    for path in FFT_SOURCES:
        h.update(open(path, "rb").read())
    out = [f"calibration (copy kernel, {cbytes} B read and written per launch): "
           f"FETCH_SIZE factor {cf:.5f}, WRITE_SIZE factor {cw:.5f}", "",
           "| stage | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes (calibrated) | "
           "algorithmic bytes | ratio |", "|---|---|---|---|---|---|"]
    per = {}
    for key, (name, nb, _) in st.items():
        if key in f and key in w:
            b = (f[key] * cf + w[key] * cw) * 1024
            per[key] = b
            out.append(f"| {name} | {f[key]:.1f} | {w[key]:.1f} | {b:.0f} | {nb} | {b / nb:.5f} |")
    out += ["", f"traffic_bytes_per_launch: {per.get(('cmul', 0), 0):.0f}",
            f"kernel_source_sha256: {h.hexdigest()}"]
    return "\n".join(out)


def counters(d: str, family: str) -> str:
    """Mean per dispatch of every collected counter, per kernel group."""
    if family == "dense":
        key, sources = (lambda r: dense_kind(r["Kernel_Name"])), DENSE_SOURCES
    elif family == "fft":
        def key(r):
            k = fft_key(r)
            return fft_stages().get(k, (f"{k[0]} {k[1]}",))[0] if k[0] != "copy" else "copy"
        sources = FFT_SOURCES
    else:
        key, sources = (lambda r: kind(r["Kernel_Name"], act_of(r["Kernel_Name"]))), SOURCES
    rows = list(csv.DictReader(open(_one(os.path.join(d, "*_counter_collection.csv")))))
    acc: dict = {}
    disp: dict = {}
    names: list = []
    for r in rows:
        k = key(r)
        if k == "other":
            continue
        c = r["Counter_Name"]
        if c not in names:
            names.append(c)
        acc.setdefault(k, {}).setdefault(c, []).append(float(r["Counter_Value"]))
        disp.setdefault(k, set()).add(r["Dispatch_Id"])
    out = ["| kernel | dispatches | " + " | ".join(names) + " |",
           "|---|---|" + "---|" * len(names)]
    for k in sorted(acc):
        vals = [f"{statistics.fmean(acc[k][c]):.6g}" if c in acc[k] else "-" for c in names]
        out.append(f"| {k} | {len(disp[k])} | " + " | ".join(vals) + " |")
    h = hashlib.sha256()
    for path in sources:
        h.update(open(path, "rb").read())
    out += ["", f"kernel_source_sha256: {h.hexdigest()}"]
    return "\n".join(out)


def main(argv):
    io, elements = IO, None
    for flag in ("--io", "--elements"):
        if flag in argv:
            i = argv.index(flag)
            if flag == "--io":
                io = argv[i + 1]
            else:
                elements = int(argv[i + 1])
            argv = argv[:i] + argv[i + 2:]
    set_io(io, elements)
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace(argv[1]))
    elif len(argv) >= 3 and argv[0] == "traffic":
        print(traffic(argv[1], argv[2]))
    elif len(argv) >= 3 and argv[0] == "dense-trace":
        print(dense_trace(argv[1], argv[2]))
    elif len(argv) >= 4 and argv[0] == "dense-traffic":
        print(dense_traffic(argv[1], argv[2], argv[3]))
    elif len(argv) >= 2 and argv[0] == "grouped-trace":
        print(grouped_trace(argv[1], int(argv[2]) if len(argv) >= 3 else 200))
    elif len(argv) >= 2 and argv[0] == "valu":
        print(valu(argv[1]))
    elif len(argv) >= 2 and argv[0] == "timeline":
        print(timeline(argv[1], int(argv[2]) if len(argv) >= 3 else 10))
    elif len(argv) >= 2 and argv[0] == "fft-trace":
        print(fft_trace(argv[1]))
    elif len(argv) >= 3 and argv[0] == "fft-traffic":
        print(fft_traffic(argv[1], argv[2]))
    elif len(argv) >= 3 and argv[0] == "counters":
        print(counters(argv[1], argv[2]))
    elif len(argv) >= 1 and argv[0] == "rare":
        print(rare_rate(int(argv[1]) if len(argv) >= 2 else 4))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
