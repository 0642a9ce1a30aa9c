"""Summarise rocprofv3 CSV output of bench.py into short markdown tables.

Usage (after the rocprofv3 runs listed in each summary's header):

    python -m memory_efficient_activation_amd.rocprof_summary trace DIR
    python -m memory_efficient_activation_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR
    python -m memory_efficient_activation_amd.rocprof_summary dense-trace DIR f32|bf16
    python -m memory_efficient_activation_amd.rocprof_summary dense-traffic FETCH_DIR WRITE_DIR f32|bf16

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
``dense-*`` the same for ``bench.py --dense`` (DenseNet-BC-100 block 1,
            layer 16: 204 channels of 64 x 32 x 32; its newest source has 12):
            forward 2 C M b bytes per launch, backward reduction 2 C M b,
            backward apply 3 C M b, statistics 12 M b, copy 2 C M b.
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
BF16 = 2                     # bytes per element
COPY_BYTES = BF16 * N        # bytes the copy kernel reads (and writes) per launch
ALGO = {"fwd": 2 * BF16 * N, "bwd": 3 * BF16 * N, "copy": 2 * BF16 * N}


ACT_NAMES = ["swish", "relu", "leaky_relu", "sigmoid", "tanh", "gelu", "gelu_tanh"]


def kind(name: str, act: str = "swish") -> str:
    """'fwd' / 'bwd' for the bf16 vector kernel of activation `act`, 'copy'
    for the copy kernel, 'other' otherwise."""
    m = re.search(r"act_vec_kernel<meswish::bf16_t, (true|false), (\d+)>", name)
    if m:
        if ACT_NAMES[int(m.group(2))] != act:
            return "other"
        return "bwd" if m.group(1) == "true" else "fwd"
    if "copy16_kernel" in name:
        return "copy"
    return "other"


def act_of(name: str) -> str:
    m = re.search(r"act_vec_kernel<meswish::bf16_t, (?:true|false), (\d+)>", name)
    return ACT_NAMES[int(m.group(1))] if m else ""


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


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace(argv[1]))
    elif len(argv) >= 3 and argv[0] == "traffic":
        print(traffic(argv[1], argv[2]))
    elif len(argv) >= 3 and argv[0] == "dense-trace":
        print(dense_trace(argv[1], argv[2]))
    elif len(argv) >= 4 and argv[0] == "dense-traffic":
        print(dense_traffic(argv[1], argv[2], argv[3]))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
