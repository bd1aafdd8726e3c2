"""bench.py's host-side contract: more than one GPU is refused before any
GPU work, and the quantization-error diagnostic it reports equals a direct
computation from the oracle's codes and scales (run here on CPU tensors)."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr and r.stdout.strip() == ""


@pytest.mark.parametrize("gran", ["tensor", "row", "1x128", "128x128"])
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_quant_rel_err_matches_direct_computation(gran, fmt):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((300, 260)) * np.exp(rng.uniform(-3, 3, (300, 1)))).astype(np.float32)
    r = oracle.quantize(x, fmt, gran)
    t = oracle.decode_table(fmt)
    R, C = x.shape
    s = r["scale_inv"].astype(np.float64)
    if gran == "tensor":
        se = np.full((R, C), s.ravel()[0])
    elif gran == "row":
        se = np.repeat(s.reshape(R, 1), C, axis=1)
    elif gran == "1x128":
        se = np.repeat(s.reshape(R, -1), 128, axis=1)[:, :C]
    else:
        se = np.repeat(np.repeat(s.reshape(-(-R // 128), -1), 128, axis=0)[:R], 128, axis=1)[:, :C]
    xh = t[r["q"]].astype(np.float64) * se
    want = np.linalg.norm(xh - x) / np.linalg.norm(x.astype(np.float64))
    got = bench.quant_rel_err(torch, torch.from_numpy(x), torch.from_numpy(r["q"]),
                              torch.from_numpy(r["scale_inv"].astype(np.float32)),
                              "e4m3" if fmt == oracle.E4M3 else "e5m2", gran)
    assert abs(got - want) <= 1e-5 * want
    gt = bench.quant_rel_err(torch, torch.from_numpy(np.ascontiguousarray(x.T)), torch.from_numpy(r["q"]),
                             torch.from_numpy(r["scale_inv"].astype(np.float32)),
                             "e4m3" if fmt == oracle.E4M3 else "e5m2", gran, transposed=True)
    assert abs(gt - want) <= 1e-5 * want


@pytest.mark.parametrize("workload", ["tiny", "mlp8b", "qkv", "mlp70b", "wgrad", "dgrad", "moe"])
def test_cpu_baseline_leg_of_every_workload(workload):
    """The CPU-oracle leg runs for every GEMM workload (small samples here)
    and reports what the bench line promises: a positive rate, the cores,
    what the sample was, and the quantize and GEMM rates on their own."""
    import types
    import synth
    args = types.SimpleNamespace(cpu_rows=32, cpu_cols=256)
    d = bench.cpu_baseline(args, workload, synth)
    assert d["kind"] == "oracle" and d["unit"] == "TFLOP/s" and d["value"] > 0 and d["cores"] >= 1
    assert d["quantize_gbs"] > 0 and d["quantize_gbs_1_thread"] > 0 and d["gemm_gflops"] > 0
    assert "GEMM" in d["sample"] and d["sample"].endswith(" s")


def test_traffic_figure_goes_stale_with_its_kernel(monkeypatch):
    """The recorded HBM bytes are reported only with the kernel source they
    were measured on."""
    b, note = bench.traffic("mlp8b")
    assert b == bench.TRAFFIC["mlp8b"]["bytes"] and "rocprofv3" in note
    monkeypatch.setitem(bench.TRAFFIC, "mlp8b", dict(bench.TRAFFIC["mlp8b"], sha16="0" * 16))
    b, note = bench.traffic("mlp8b")
    assert b is None and note.startswith("stale")
    assert bench.traffic("tiny")[0] is None
