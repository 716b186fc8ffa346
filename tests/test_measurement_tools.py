"""The measurement plumbing on the CPU: the counter summary that turns
rocprofv3 FETCH_SIZE / WRITE_SIZE rows into HBM bytes per call (calibrated
by the plain device copy of known size), and bench.py's reader, which takes
a recorded figure only while the kernel source still hashes to the one the
counters were taken on."""
import csv
import hashlib
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY = "__amd_rocclr_copyBuffer"
FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value})


def _summary(tmp_path, fetch_rows, write_rows, copy_bytes=512 << 20):
    src = tmp_path / "kernel.hip"
    src.write_text("// a kernel source\n")
    fetch, write, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.md"
    _csv(fetch, "FETCH_SIZE", fetch_rows)
    _csv(write, "WRITE_SIZE", write_rows)
    r = subprocess.run([sys.executable, "rocprof_summary.py", "traffic",
                        "--fetch", str(fetch), "--write", str(write),
                        "--copy-bytes", str(copy_bytes), "--kernel", "gemm_i8_kernel",
                        "--source", str(src), "--workload", "test",
                        "--algorithmic-bytes", "1e6", "--command-fetch", "cf",
                        "--command-write", "cw", "-o", str(out)],
                       cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    fields = dict(line.split(": ", 1) for line in out.read_text().splitlines()
                  if line.endswith(tuple("0123456789abcdef")) and ": " in line
                  and not line.startswith(("|", "Calibration")))
    return fields, src


def test_traffic_is_calibrated_and_summed_over_instantiations(tmp_path):
    """FETCH_SIZE of the copy reads half its bytes (scale 2), WRITE_SIZE all
    of them (scale 1).  The GEMM's main launch (two dispatches, averaged) and
    its tail launch (another instantiation) add up to one call; kernels that
    do not match are ignored."""
    fetch = [(COPY, 262144.0), (COPY, 262144.0),
             ("void gemm_i8_kernel<1, false, 4, 4>(...)", 1000.0),
             ("void gemm_i8_kernel<1, false, 4, 4>(...)", 1200.0),
             ("void gemm_i8_kernel<1, false, 2, 4>(...)", 100.0),
             ("void rotquant_stream_kernel<1, 128>(...)", 9999.0)]
    write = [(COPY, 524288.0),
             ("void gemm_i8_kernel<1, false, 4, 4>(...)", 300.0),
             ("void gemm_i8_kernel<1, false, 2, 4>(...)", 20.0)]
    f, src = _summary(tmp_path, fetch, write)
    read = (1100.0 + 100.0) * 1024 * 2.0
    wrote = (300.0 + 20.0) * 1024 * 1.0
    assert float(f["read_bytes_per_launch"]) == read
    assert float(f["write_bytes_per_launch"]) == wrote
    assert float(f["traffic_bytes_per_launch"]) == read + wrote
    assert f["kernel_source_sha256"] == hashlib.sha256(src.read_bytes()).hexdigest()


def test_traffic_without_a_matching_kernel_fails(tmp_path):
    fetch = [(COPY, 262144.0), ("void other_kernel(...)", 5.0)]
    write = [(COPY, 524288.0), ("void other_kernel(...)", 5.0)]
    src = tmp_path / "kernel.hip"
    src.write_text("x")
    _csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    r = subprocess.run([sys.executable, "rocprof_summary.py", "traffic",
                        "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
                        "--copy-bytes", "1", "--kernel", "gemm_i8_kernel", "--source", str(src),
                        "--workload", "t", "--command-fetch", "a", "--command-write", "b"],
                       cwd=ROOT, capture_output=True, text=True)
    assert r.returncode != 0 and "no dispatch" in (r.stderr + r.stdout)


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_recorded_traffic_only_for_the_current_source(tmp_path, monkeypatch):
    bench = _bench()
    src = tmp_path / "gemm_i8.hip"
    src.write_text("// version 1\n")
    (tmp_path / "profiles").mkdir()
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    (tmp_path / "profiles" / "gemm_i8_w_pmc.md").write_text(
        f"traffic_bytes_per_launch: 6.5e+09\nkernel_source_sha256: {sha}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "SOURCES", {"gemm_i8": str(src)})
    assert bench.recorded_traffic("gemm_i8", "w") == 6.5e9
    assert bench.recorded_traffic("gemm_i8", "other_workload") is None
    src.write_text("// version 2\n")                  # the kernel changed since
    assert bench.recorded_traffic("gemm_i8", "w") is None

