"""Host-side parts of bench.py (no GPU): the trace and traffic summaries it
computes from rocprofv3 output, and the refusal of more than one GPU."""
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


def test_traffic_summary_and_its_use(tmp_path):
    """The traffic file: each counter scaled by the copy kernel's reading of
    the known weight bytes, and bench.py takes its figure only for the same
    kernel sources and the same planned variant."""
    sys.path.insert(0, ROOT)
    import bench

    wl, t = "q8_0_4096x4096", 1
    wb = bench.WEIGHT_BYTES[wl]
    # the copy reads 2x the bytes it copies (scale 0.5) and writes them once
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    kname = "void qmv::k_flat<0, 1, 1, 2, 4, true, 8, false, 0, false>(qmv::StreamArgs)"
    with open(fetch, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for _ in range(3):
            f.write(f"__amd_rocclr_copyBuffer,FETCH_SIZE,{2 * wb / 1024}\n")
        for v in (1.0, 3.0, 2.0):  # median 2 x the weight bytes
            f.write(f"\"{kname}\",FETCH_SIZE,{v * wb / 1024}\n")
        f.write("qmv::k_quantize(float const*),FETCH_SIZE,99\n")
    with open(write, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        f.write(f"__amd_rocclr_copyBuffer,WRITE_SIZE,{wb / 1024}\n")
        f.write(f"\"{kname}\",WRITE_SIZE,16.0\n")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--traffic-summary", str(fetch), str(write),
                        "--workload", wl, "--tokens", str(t)], capture_output=True, text=True, check=True)
    text = r.stdout
    assert f"# kernel: {kname}" in text
    expect = wb + 16 * 1024  # reads: median 2 x wb scaled by 0.5; writes: 16 KiB at scale 1
    line = [x for x in text.splitlines() if x.startswith("traffic_bytes_per_launch:")][0]
    assert abs(float(line.split()[1]) - expect) < 2
    variant = [x for x in text.splitlines() if x.startswith("matvec_variant:")][0].split()[1]
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / f"traffic_{wl}_t{t}.txt").write_text(text)
    old_root = bench.ROOT
    try:
        bench.ROOT = str(tmp_path)
        src = [x for x in text.splitlines() if x.startswith("kernel_sources_sha256_16:")][0].split()[1]
        assert bench.recorded_traffic(wl, t, src, variant) == float(line.split()[1])
        assert bench.recorded_traffic(wl, t, "0" * 16, variant) is None      # other kernel sources
        assert bench.recorded_traffic(wl, t, src, "lpr64_r2") is None        # another variant
        assert bench.recorded_traffic(wl, 2, src, variant) is None           # no file
    finally:
        bench.ROOT = old_root
