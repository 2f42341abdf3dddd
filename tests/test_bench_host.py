"""Host-side checks of bench.py: the one-GPU guard and the trace summary's
selection of timed calls (no GPU needed)."""

import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_trace(path, n_calls, split_us, merge_us):
    """A kernel-trace CSV of n_calls calls (one split, then one merge dispatch each),
    in rocprofv3's column names; the rows are written out of order."""
    rows, t = [], 1_000_000
    for i in range(n_calls):
        s0, s1 = t, t + int(split_us(i) * 1e3)
        m0, m1 = s1 + 500, s1 + 500 + int(merge_us(i) * 1e3)
        rows.append({"Kernel_Name": "va::split_kernel(va::SplitArgs)", "Start_Timestamp": s0, "End_Timestamp": s1})
        rows.append({"Kernel_Name": "va::merge_kernel(...)", "Start_Timestamp": m0, "End_Timestamp": m1})
        rows.append({"Kernel_Name": "void at::native::reduce_kernel<...>", "Start_Timestamp": m1 + 10,
                     "End_Timestamp": m1 + 20})
        t = m1 + 100_000
    rows.reverse()
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)


def _row(text, kernel, kind):
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip("|").split("|")]
        if len(cells) == 6 and cells[0] == kernel and cells[2] == kind:
            return int(cells[1]), float(cells[3]), float(cells[4]), float(cells[5])
    raise AssertionError(f"no row for {kernel} {kind}")


def test_trace_summary_takes_the_timed_steps_only(tmp_path):
    warmup, steps = 3, 5           # steps of four calls each
    first = 4 * warmup

    # Warmup calls take 1000 us; timed call k (k = 0..4*steps-1) takes 100 + (k % 4) + 10 * (k // 4),
    # so the cold calls (k % 4 in {0, 1}) and warm calls ({2, 3}) have known averages.
    def split_us(i):
        if i < first:
            return 1000.0
        k = i - first
        return 100.0 + (k % 4) + 10.0 * (k // 4)

    path = tmp_path / "trace.csv"
    _write_trace(path, first + 4 * steps, split_us, lambda i: 5.0)
    text = bench.summarize_trace(str(path), "tiny", warmup, steps)
    assert f"the first {first} calls ({warmup} warmup steps)" in text
    n, avg, lo, hi = _row(text, "split_kernel", "cold")
    assert n == 2 * steps
    assert avg == pytest.approx(100.5 + 10.0 * (steps - 1) / 2, abs=0.01)
    assert lo == pytest.approx(100.0, abs=0.01) and hi == pytest.approx(101.0 + 10.0 * (steps - 1), abs=0.01)
    n, avg, _, _ = _row(text, "split_kernel", "warm")
    assert n == 2 * steps and avg == pytest.approx(102.5 + 10.0 * (steps - 1) / 2, abs=0.01)
    n, avg, _, _ = _row(text, "merge_kernel", "cold")
    assert n == 2 * steps and avg == pytest.approx(5.0, abs=0.01)


def test_trace_summary_rejects_a_trace_of_another_command(tmp_path):
    path = tmp_path / "trace.csv"
    _write_trace(path, 4 * 3 + 4 * 5 - 1, lambda i: 100.0, lambda i: 5.0)
    with pytest.raises(SystemExit, match="expected 32 split and merge dispatches"):
        bench.summarize_trace(str(path), "tiny", 3, 5)
