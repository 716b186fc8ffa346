"""bench.py's output contract: one JSON line on stdout carrying the fields the
harness reads, the roofline entry of the dominant kernel and the oracle's
staged CPU baseline; and its refusal to run on more than one GPU."""
import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(args, timeout):
    return subprocess.run([sys.executable, "bench.py", *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_refuses_more_than_one_gpu():
    """The path shards along tokens with no exchange; the benchmark measures
    one GPU and says so when asked for more (checked before any GPU work)."""
    r = _bench(["--gpus", "2"], 300)
    assert r.returncode == 2, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


@pytest.mark.gpu
def test_json_line_contract():
    """A short run of the small workload: exactly one JSON line, the step
    count and warm-up it was given, a value consistent with its own step
    time, a roofline whose fraction is achieved / peak, the oracle baseline
    with its thread count, and no mismatch on the parity sample."""
    print("[case] bench.py --workload tiny --steps 3 --warmup 2", flush=True)
    r = _bench(["--workload", "tiny", "--steps", "3", "--warmup", "2", "--no-ceilings",
                "--cpu-seconds", "1"], 600)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])

    assert isinstance(d["metric"], str) and d["metric"]
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["higher_is_better"] is True
    assert d["scaling"] in ("weak", "strong")
    assert d["vs_baseline"] is None
    assert d["dtype"] == "int8" and d["data"] == "synthetic"
    assert d["config"]["workload"] == "tiny"
    assert "model" not in d["config"]

    # value: whole-job effective INT8 TOPS of the timed steps
    M, K, N = 256, 512, 512
    assert d["ms_per_step"] > 0
    assert math.isclose(d["value"], 2.0 * M * N * K / (d["ms_per_step"] * 1e-3) / 1e12,
                        rel_tol=0.02)

    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert roof["unit"] in ("GB/s", "TFLOP/s")
    assert roof["achieved"] > 0 and roof["peak"] > 0
    assert math.isclose(roof["frac"], roof["achieved"] / roof["peak"], rel_tol=0.01,
                        abs_tol=1e-4)
    assert roof["traffic"] is None or roof["traffic"] > 0

    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle"
    assert cpu["value"] > 0 and cpu["cores"] >= 1
    assert isinstance(cpu["unit"], str) and isinstance(cpu["sample"], str)

    assert d["parity_sample"]["mismatches"] == 0
