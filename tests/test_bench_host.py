"""Host-side parts of bench.py (no GPU): the trace summary it computes from a
rocprofv3 kernel trace, and the refusal of more than one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_trace_summary_median(tmp_path):
    # two kernels: durations 1, 2, 3, 10 us and 5, 7 us (timestamps in ns)
    rows = [("k_a", 0, 1000), ("k_a", 5000, 7000), ("k_b", 8000, 13000), ("k_a", 20000, 23000),
            ("k_a", 30000, 40000), ("k_b", 50000, 57000)]
    csv = tmp_path / "kernel_trace.csv"
    with open(csv, "w") as f:
        f.write("Kind,Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for name, s, e in rows:
            f.write(f"KERNEL_DISPATCH,{name},{s},{e}\n")
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--trace-summary", str(csv)],
                         capture_output=True, text=True, check=True).stdout.splitlines()
    table = {line.split()[-1]: line.split()[:5] for line in out[1:]}
    assert table["k_a"] == ["4", "2.500", "4.000", "1.000", "10.000"]
    assert table["k_b"] == ["2", "6.000", "6.000", "5.000", "7.000"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
