"""Host logic of bench.py that needs no GPU: the rocprofv3 summary helpers and the
settle loop."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_stats_splits_by_preceding_dispatch(tmp_path, capsys):
    """Dispatches of kernel B after kernel A count as in the step, after B itself as
    back to back; each side's median is reported."""
    _write(tmp_path / "run_kernel_stats.csv",
           ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
           [["kA", 10, 1000, 900, 1100, 20.0], ["kB", 30, 5000, 4000, 9000, 80.0]])
    trace = []
    t = 0
    # ten steps of A then B (B in the step: 4 us), then twenty B back to back (6 us)
    for _ in range(10):
        trace.append(["kA", t, t + 1000])
        t += 1000
        trace.append(["kB", t, t + 4000])
        t += 4000
    for _ in range(20):
        trace.append(["kB", t, t + 6000])
        t += 6000
    _write(tmp_path / "run_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           trace)
    bench.summarize_stats(str(tmp_path), "synthetic", tail=5)
    out = capsys.readouterr().out
    lines = [ln.split() for ln in out.splitlines() if ln.startswith("kB")]
    # the stats table, the last-5 table, the split table
    assert len(lines) == 3, out
    split = lines[-1]
    assert split[1:] == ["10", "4.00", "20", "6.00"], split
    last = lines[1]
    assert last[1:] == ["5", "6.00"], last


def test_settle_runs_for_the_set_time(monkeypatch):
    calls = []

    class FakeCuda:
        @staticmethod
        def synchronize():
            calls.append("sync")

    class FakeTorch:
        cuda = FakeCuda

    monkeypatch.setattr(bench, "SETTLE_MS", 30.0)
    t0 = bench.time.perf_counter()
    bench.settle(FakeTorch, lambda: calls.append("replay"))
    el = (bench.time.perf_counter() - t0) * 1e3
    assert el >= 30.0
    assert calls.count("replay") == 8 * calls.count("sync") > 0


@pytest.mark.parametrize("ms", [0.0])
def test_settle_zero_is_a_no_op(monkeypatch, ms):
    monkeypatch.setattr(bench, "SETTLE_MS", ms)

    class FakeTorch:
        class cuda:
            @staticmethod
            def synchronize():
                raise AssertionError("no replay expected")

    bench.settle(FakeTorch, lambda: (_ for _ in ()).throw(AssertionError("no replay")))
