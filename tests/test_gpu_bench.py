"""bench.py on the GPU, in a process of its own: its one JSON line carries
every field the benchmark contract names, with the roofline and the
kernels' figures consistent with each other (a short run of the small
workload and of the KV workload)."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}


@pytest.fixture(autouse=True)
def _need_gpu(gpu):
    yield


def _run(*args):
    say("bench", *args)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


@pytest.mark.timeout(300)
def test_bench_line_contract_tiny():
    d = _run("--workload", "tiny", "--steps", "5", "--warmup", "2", "--no-cpu-baseline", "--config-steps", "2")
    assert KEYS <= set(d) and d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    # the clock probe ran (amd-smi may find no fully busy sample for so small a GEMM)
    clk = d["kernels"]["gemm_clock_mhz"]
    assert clk is None or 300.0 <= clk <= 3000.0, clk
    assert d["higher_is_better"] is True and d["vs_baseline"] is None and "workload" in d["config"]
    roof = d["roofline"]
    assert {"bound", "achieved", "peak", "unit", "frac", "traffic"} <= set(roof)
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 5000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    k = d["kernels"]
    flops = 2.0 * 256 ** 3
    assert abs(roof["achieved"] - flops / (k["gemm_ms"] * 1e-3) / 1e12) <= 0.01 * roof["achieved"] + 0.01
    assert k["gemm_ms_back_to_back"] > 0 and "in step" not in roof["time"] and "two events" in roof["time"]
    assert abs(d["value"] - flops / (d["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * d["value"] + 0.01
    assert set(k["quantize_rel_err"]) == {"X", "W"} and 0 < k["quantize_rel_err"]["X"]["rel_err"] < 0.05
    c = k["stream_ceilings"]
    assert 0 < c["copy_gbs"] <= c["read_gbs"] * 1.05 and c["read2_write1_gbs"] > 0 and d["cpu_baseline"] is None
    assert abs(k["quantize_pct_read2_write1_ceiling"] - 100 * k["quantize_gbs"] / c["read2_write1_gbs"]) < 0.05
    assert "time" in roof and roof["traffic"] is None     # no counters for the tiny workload
    # every other GEMM workload timed in the same run, with consistent figures
    w = k["workloads"]
    assert set(w) == {"qkv", "mlp70b", "wgrad", "dgrad", "moe"}
    for name, b in w.items():
        fl = 2.0 * b["M"] * b["N"] * b["K"]
        assert abs(b["gemm_tflops"] - fl / (b["gemm_ms"] * 1e-3) / 1e12) <= 0.01 * b["gemm_tflops"] + 0.01, name
        assert abs(b["gemm_frac_fp8_peak"] - b["gemm_tflops"] / 5000.0) < 1e-3, name
        assert b["step_ms"] > 0 and b["quantize_ms"] > 0, name
    assert (w["mlp70b"]["M"], w["mlp70b"]["N"], w["mlp70b"]["K"]) == (2048, 28672, 8192)


@pytest.mark.timeout(300)
def test_bench_line_contract_kv():
    d = _run("--workload", "kv", "--steps", "5", "--warmup", "2", "--no-cpu-baseline")
    assert KEYS <= set(d) and d["unit"] == "GB/s" and d["n_gpus"] == 1
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
