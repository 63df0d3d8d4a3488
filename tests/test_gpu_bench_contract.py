"""The benchmark's output line on the GPU, from a short run of the default
workload (c2): one JSON line with the fields the contract names, and their
relations: value is the algorithmic bytes of a decode step over its time, the
roofline describes the decode kernel (its bytes per launch over its mean
launch time from the library's timing events), and frac is achieved over the
8 TB/s HBM peak."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from kv_cache_bit_kivi_amd.inputs import WORKLOADS  # noqa: E402

pytestmark = pytest.mark.gpu


def test_bench_line_contract():
    print("bench: c2, 6 steps, 1 warm-up, no CPU baseline", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "6",
                        "--warmup", "1", "--cold-iters", "2", "--pack-iters", "1", "--probe-iters", "2",
                        "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-3000:]
    j = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in j, k
    assert (j["n_gpus"], j["steps"], j["warmup"]) == (1, 6, 1)
    assert j["unit"] == "GB/s" and j["higher_is_better"] is True and j["data"] == "synthetic"
    assert j["vs_baseline"] is None and j["cpu_baseline"] is None
    assert j["dtype"] == "f16"  # the decode's matrix-product operand type
    assert j["config"]["workload"].startswith("c2:")
    ab = bench.algorithmic_bytes(WORKLOADS["c2"])
    assert j["value"] == pytest.approx(bench.step_bytes(ab) / (j["ms_per_step"] * 1e-3) / 1e9, rel=1e-9)
    rf = j["roofline"]
    for k in ("bound", "kernel", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert (rf["bound"], rf["kernel"], rf["peak"], rf["unit"]) == ("hbm", "decode_mfma", 8000.0, "GB/s")
    assert rf["bytes_per_launch"] == ab["decode"]
    assert rf["achieved"] == pytest.approx(rf["bytes_per_launch"] / (rf["us_per_launch"] * 1e-6) / 1e9,
                                           rel=1e-9)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-12)
    assert 0.0 < rf["frac"] < 1.0
    ph = j["phases"]
    assert ph["decode"]["samples"] == 3 and ph["decode"]["us_mean"] == pytest.approx(rf["us_per_launch"])
    # the decode kernel is the step's largest part; flush and merge are short
    assert ph["decode"]["us_mean"] > ph["flush"]["us_mean"] and ph["decode"]["us_mean"] > ph["merge"]["us_mean"]
    assert 0.0 < ph["stream_read_probe"]["frac"] < 1.0
    assert rf["frac_of_stream_read"] == pytest.approx(rf["achieved"] / ph["stream_read_probe"]["gbps"])
    # null when the kernel source changed after the counters were taken;
    # otherwise the measured HBM bytes are close to the algorithmic ones
    if rf["traffic"] is not None:
        assert 0.95 <= rf["traffic"] / rf["bytes_per_launch"] <= 1.2
