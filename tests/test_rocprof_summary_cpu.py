"""The profile summariser (memory_efficient_activation_amd/rocprof_summary.py)
on synthetic rocprofv3 CSV files: region detection and the per-window means
of ``timeline`` and ``grouped-trace``, whose tables stand in profiles/."""

import csv

import pytest

from memory_efficient_activation_amd import rocprof_summary as rs

FWD = "void meswish::act_vec_kernel<meswish::bf16_t, false, 0>(meswish::bf16_t const*, x)"
BWD = "void meswish::act_vec_kernel<meswish::bf16_t, true, 0>(meswish::bf16_t const*, x)"
COPY = "meswish::copy16_kernel(HIP_vector_type<unsigned int, 4u> const*, x)"
GF = "void meswish::act_group_kernel<meswish::bf16_t, false, 0>(meswish::GroupArgs, meswish::Coef)"
GB = "void meswish::act_group_kernel<meswish::bf16_t, true, 0>(meswish::GroupArgs, meswish::Coef)"
OTHER = "void at::native::elementwise_kernel<128, 4>(int, x)"


def _write_trace(d, launches):
    """launches: (name, duration in ns); back to back with 1 us gaps."""
    t = 1_000_000
    with open(d / "trace_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Dispatch_Id"])
        for i, (name, dur) in enumerate(launches):
            w.writerow([name, t, t + dur, i + 1])
            t += dur + 1000
    names = sorted({n for n, _ in launches})
    with open(d / "trace_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        for n in names:
            ds = [x for m, x in launches if m == n]
            w.writerow([n, len(ds), sum(ds), sum(ds) / len(ds), 0, min(ds), max(ds), 0])


def _rows(table):
    return [[c.strip() for c in line.strip("|").split("|")] for line in table.splitlines()[2:]]


def test_timeline_regions_and_means(tmp_path):
    # 30 alternating steps (fwd 40 us, bwd 60 us, the last 10 slower), then
    # 12 backward and 12 forward launches back to back, then 5 copies; an
    # unrelated kernel in between is ignored.
    seq = []
    for i in range(30):
        slow = 10_000 if i >= 20 else 0
        seq += [(FWD, 40_000 + slow), (BWD, 60_000 + slow)]
    seq += [(OTHER, 5_000)] + [(BWD, 62_000)] * 12 + [(FWD, 42_000)] * 12 + [(COPY, 41_000)] * 5
    _write_trace(tmp_path, seq)
    rows = _rows(rs.timeline(str(tmp_path), 10))
    labels = [(r[0], int(r[1])) for r in rows]
    assert labels == [("swish fwd/bwd", 20), ("swish fwd/bwd", 20), ("swish fwd/bwd", 20),
                      ("swish bwd", 10), ("swish bwd", 2), ("swish fwd", 10), ("swish fwd", 2),
                      ("copy", 5)]
    assert rows[0][3:5] == ["40.0", "60.0"] and rows[2][3:5] == ["50.0", "70.0"]
    # Step rate of the first window: 10 steps of 10 B n per 100 us.
    assert int(rows[0][6]) == round(10 * (rs.ALGO["fwd"] + rs.ALGO["bwd"]) / 1_000_000)
    assert rows[3][4] == "62.0" and rows[5][3] == "42.0" and rows[7][5] == "41.0"


def test_grouped_trace_regions(tmp_path):
    seq = []
    for _ in range(60):
        seq += [(GF, 46_000), (GB, 63_000)]
    seq += [(GB, 68_000)] * 20 + [(GF, 46_500)] * 20
    for _ in range(4):
        seq += [(FWD, 5_000)] * 7 + [(BWD, 7_000)] * 7
    _write_trace(tmp_path, seq)
    rows = _rows(rs.grouped_trace(str(tmp_path), steps=50).split("\n\n")[1])
    got = {r[0]: (int(r[1]), float(r[2])) for r in rows}
    assert got["grouped forward, timed alternating steps"] == (50, 46.0)
    assert got["grouped backward, timed alternating steps"] == (50, 63.0)
    assert got["grouped backward only, back to back"] == (20, 68.0)
    assert got["grouped forward only, back to back"] == (20, 46.5)
    assert got["single launches, 14 per step (kernel time per step)"] == (56, 84.0)
    gbps = {r[0]: int(r[3]) for r in rows}
    assert gbps["grouped backward only, back to back"] == round(6 * rs.GROUPED_ELEMS / 68_000)


def test_one_file_per_pattern(tmp_path):
    with pytest.raises(SystemExit):
        rs.timeline(str(tmp_path))


def test_valu_table(tmp_path):
    names = {"fwd": FWD, "bwd": BWD}
    with open(tmp_path / "valu_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        n = rs.N
        for i, (k, busy, per) in enumerate([("fwd", 30.0, 9), ("bwd", 40.0, 15), ("bwd", 50.0, 15)]):
            for c, v in (("VALUBusy", busy), ("SQ_INSTS_VALU", per * n / 64),
                         ("SQ_INSTS_VALU_TRANS_F32", 2 * n / 64), ("SQ_WAVES", n / 512)):
                w.writerow([i + 1, names[k], c, v, 0, 60_000])
    rows = {r[0]: r for r in _rows(rs.valu(str(tmp_path)))}
    assert rows["swish fwd"][1:] == ["1", "60.0", "30.0", "9.00", "2.00"]
    assert rows["swish bwd"][1:] == ["2", "60.0", "45.0", "15.00", "2.00"]


def test_counters_table(tmp_path):
    """Means per dispatch per kernel group, one column per counter, in the
    order the counters first appear; unrelated kernels are left out."""
    fwd = "void dense_bn::fwd_kernel<float, 4>(dense_bn::Table, x)"
    with open(tmp_path / "u_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name",
                    "Counter_Value"])
        for d, (name, a, b) in enumerate([(fwd, 10, 1), (fwd, 30, 3), (COPY, 7, 2),
                                          (OTHER, 99, 99)]):
            w.writerow([d + 1, name, 256, 256, "A_CTR", a])
            w.writerow([d + 1, name, 256, 256, "B_CTR", b])
    rows = _rows(rs.counters(str(tmp_path), "dense"))
    assert rows[0] == ["copy", "1", "7", "2"]
    assert rows[1] == ["fwd", "2", "20", "2"]
    assert len([r for r in rows if r and r[0] in ("copy", "fwd")]) == 2
