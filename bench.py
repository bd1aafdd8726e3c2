#!/usr/bin/env python3
"""Benchmark of the FP8 hot path on one MI355X.

One step = the whole path over one batch of seeded synthetic input already
resident in HBM: amax + scale + saturating RNE cast of both GEMM operands,
then the scaled FP8 GEMM with fp32 accumulation and its dequantizing
epilogue.  Default workload: the 8B-style MLP up-projection
(X [4096 x 4096] bf16 with 0.1% outlier columns x50, W [14336 x 4096] bf16
N(0, 0.02), per-tensor dynamic E4M3 scaling, Y bf16).

Prints ONE JSON line.  `value` = whole-step throughput in TFLOP/s
(2MNK / step time); the GEMM's own TFLOP/s and % of the FP8 MFMA peak, and
the quantize GB/s and % of HBM peak, are in `kernels` and `roofline`.  The
K steps are timed as a whole by two HIP events around the loop (an event
recorded between kernels costs the GPU several microseconds of idle time,
so none is); the GEMM's and the quantize's own times come from K calls of
each back to back, and their per-step spreads from a further K steps with
events around each operation.  In a step the quantize also pays for the
write-back of the previous GEMM's output from the cache, so its share of a
step (step minus GEMM) is reported beside its own time.  After
the timed steps, `kernels` also gets the graphics clock sampled (amd-smi)
while the GEMM repeats for 1.5 s, the GEMM's % of the FP8 peak at that
clock, and hand-written streaming probes (read-only, copy, and 16 bytes read
per 8 written, the cast's own pattern) as the practical HBM ceilings of the
quantize; per-step times come as mean and as
median / p10 / p90; `quantize_rel_err` is each operand's ||dequant(q) - x|| /
||x|| with its granularity and format.  `cpu_baseline` is the oracle on a bounded sample of
the same step (quantize on all threads and on one, GEMM on all threads).

    python bench.py [--steps K] [--warmup W] [--workload mlp8b|qkv|mlp70b|wgrad|dgrad|moe|kv|tiny]

The kv workload is the memory-bound FP8 KV cache instead (its own JSON line
in GB/s): one step = one layer's store of a 8192-token chunk of K and V into
E4M3 caches through a page table, then the gather-dequantize of the whole
32768-token context to bf16.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
# rocprofv3 HBM traffic of one call of the roofline kernel: FETCH_SIZE x 2.0 +
# WRITE_SIZE x 1.0 per dispatch (factors from a plain 512 MiB copy), with the
# first 16 hex digits of the sha256 of the kernel source the counters were
# taken with.  A run whose source differs reports no traffic (null) and says
# the figure is stale, until the counters are taken again.
#   mlp8b: one scaled-GEMM call (profiles/k_gemm_mlp8b_hbm_traffic.md)
#   kv: one fp8_kv_load launch (profiles/kv_store_gather_8x128_paged_kernel_stats.md)
TRAFFIC = {
    "mlp8b": {"bytes": 504843973, "source": "csrc/gemm.hip", "sha16": "0a8746efb4236bf4"},
    "kv": {"bytes": 104882176, "source": "csrc/kvcache.hip", "sha16": "119ccf3371e008a4"},
}


def traffic(workload: str):
    """(bytes, note): the recorded HBM bytes of the roofline kernel when its
    source is the one the counters were taken with, else (None, why)."""
    import hashlib
    t = TRAFFIC.get(workload)
    if t is None:
        return None, "no counters taken for this workload"
    path = os.path.join(ROOT, "fp8_precision_quantization_amd", t["source"])
    sha = hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]
    if sha != t["sha16"]:
        return None, "stale: %s changed since the counters were taken (%s, now %s)" % (t["source"], t["sha16"], sha)
    return t["bytes"], "rocprofv3 FETCH_SIZE/WRITE_SIZE with %s at %s" % (t["source"], sha)

WORKLOADS = {
    "tiny": "tiny: X, W [256 x 256] fp32 N(0,1); per-tensor E4M3; Y fp32",
    "mlp8b": ("mlp8b: X [4096 x 4096] bf16 N(0,1) with 0.1% outlier columns x50, "
              "W [14336 x 4096] bf16 N(0,0.02); per-tensor dynamic E4M3; Y bf16"),
    "qkv": ("qkv: X [8192 x 4096] bf16 with outlier columns, W [6144 x 4096] bf16; "
            "row-wise power-of-two scales, E4M3; Y bf16"),
    "mlp70b": ("mlp70b: X [2048 x 8192] bf16 Student-t(4) 1x128 blocks, W [28672 x 8192] bf16 "
               "N(0,0.015) 128x128 blocks, E4M3; block-scaled GEMM; Y bf16"),
    "wgrad": ("wgrad: dY [8192 x 4096] bf16 1e-3*t(3) -> E5M2, X [8192 x 4096] bf16 N(0,1) -> E4M3, "
              "delayed scaling (16-step history), transposed casts; dW = dY^T X [4096 x 4096] fp32"),
    "dgrad": ("dgrad: dY [4096 x 14336] bf16 1e-3*t(3) -> E5M2 delayed, both layouts in one pass; "
              "W [14336 x 4096] bf16 N(0,0.02) -> E4M3 transposed; dX = dY W [4096 x 4096] bf16"),
    "moe": ("moe: Mixtral-style expert up-projection, 8 experts, 4096 tokens routed top-2 (8192 rows, "
            "uneven expert loads); routed X [8192 x 4096] bf16 cast row-wise to E4M3 each step; expert W "
            "[8 x 14336 x 4096] E4M3 per-tensor per expert (cast once); grouped GEMM, Y bf16"),
    "kv": ("kv: one layer of an 8B-style model, 8 KV heads x 128; K (outlier channels) and V bf16 of a "
           "8192-token chunk stored as E4M3 with per-(token, head) scales into 32768-row caches through "
           "a 16-row page table, then all 32768 rows of K and V gathered and dequantized to bf16; "
           "4 layers rotate"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mlp8b", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="X rows in the CPU-baseline sample (default: all of mlp8b's, about 10-15 s on 16 cores)")
    ap.add_argument("--cpu-cols", type=int, default=14336, help="W rows in the CPU-baseline sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for the HBM byte counters)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the 1.5 s GEMM loop that samples the graphics clock")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload block (the other GEMM workloads timed in the same run)")
    ap.add_argument("--config-steps", type=int, default=20,
                    help="back-to-back calls per operation in the per-workload block")
    return ap.parse_args()


def phase(torch, name: str):
    """A named range (roctx on ROCm, through torch's nvtx module) around a
    phase of the run, visible in rocprofv3's marker trace; a no-op where the
    module is unavailable."""
    import contextlib
    try:
        return torch.cuda.nvtx.range(name)
    except Exception:
        return contextlib.nullcontext()


def loop_ms(torch, fn, n: int) -> float:
    """Mean ms per call of fn over n calls back to back, timed by two HIP
    events around the whole loop (nothing else on the stream between the
    calls: a HIP event recorded between kernels costs the GPU several
    microseconds of idle time here)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def quant_rel_err(torch, x, q, s_inv, fmt: str, gran: str, transposed: bool = False) -> float:
    """Relative error ||dequant(q) - x|| / ||x|| (Frobenius) of one cast,
    on the GPU with torch: codes decoded through torch's own float8 view of
    all 256 codes, times each element's group scale_inv."""
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    table = torch.arange(256, dtype=torch.uint8).view(dt).to(torch.float32).to(q.device)
    xf = x.to(torch.float32)
    if transposed:
        xf = xf.t()
    R, C = xf.shape
    if gran == "tensor":
        s = s_inv.reshape(1, 1)
    elif gran == "row":
        s = s_inv.reshape(R, 1)
    elif gran == "1x128":
        s = s_inv.reshape(R, -1).repeat_interleave(128, dim=1)[:, :C]
    else:
        s = s_inv.reshape(-(-R // 128), -1).repeat_interleave(128, dim=0)[:R].repeat_interleave(128, dim=1)[:, :C]
    err = (table[q.long()] * s - xf).norm() / xf.norm()
    return float(err)


def spread(ms):
    """Median, p10 and p90 of per-step times (ms)."""
    return {"median": round(float(np.median(ms)), 4), "p10": round(float(np.percentile(ms, 10)), 4),
            "p90": round(float(np.percentile(ms, 90)), 4)}


def stream_ceilings(torch, mib: int = 1024, reps: int = 5, rounds: int = 3) -> dict:
    """HBM ceilings from the hand-written streaming probes (libfp8probe.so):
    a read-only stream, a copy, and 16 bytes read per 8 written (a bf16 ->
    FP8 cast's pattern without its arithmetic), each over `mib` MiB of
    source alternating between two buffers (so nothing is left in the
    256 MB Infinity Cache), the best of `rounds` rounds of `reps` launches;
    GB/s of bytes read + written.  For each, the best of 2, 4 and 8
    workgroups per CU (each workgroup streaming one contiguous run)."""
    import ctypes
    path = os.path.join(ROOT, "fp8_precision_quantization_amd", "libfp8probe.so")
    if not os.path.exists(path):
        raise ImportError("libfp8probe.so is not built at %s" % path)
    L = ctypes.CDLL(path)
    P, I64, INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.fp8probe_read.argtypes = [P, I64, P, I64, INT, P]
    L.fp8probe_copy.argtypes = [P, P, I64, INT, P]
    L.fp8probe_read2_write1.argtypes = [P, P, I64, INT, P]
    n = mib * 2 ** 20
    src = [torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(i + 1) for i in range(2)]
    dst = [torch.empty(n, dtype=torch.uint8, device="cuda:0") for _ in range(2)]
    sink = torch.empty(1 << 16, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    launches = {
        "read": (lambda i, b: L.fp8probe_read(src[i].data_ptr(), n, sink.data_ptr(), sink.numel(), b, stream), n),
        "copy": (lambda i, b: L.fp8probe_copy(src[i].data_ptr(), dst[i].data_ptr(), n, b, stream), 2 * n),
        "read2_write1": (lambda i, b: L.fp8probe_read2_write1(src[i].data_ptr(), dst[i].data_ptr(), n, b, stream),
                         n + n // 2),
    }
    out = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, (run, nbytes) in launches.items():
        best = 0.0
        for bpc in (2, 4, 8):
            for i in range(2):
                if run(i, bpc) != 0:
                    raise RuntimeError("fp8probe %s failed" % name)
            torch.cuda.synchronize()
            for _ in range(rounds):
                e0.record()
                for r in range(reps):
                    run(r & 1, bpc)
                e1.record()
                torch.cuda.synchronize()
                best = max(best, nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        out[name + "_gbs"] = round(best, 1)
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


def gemm_clock_mhz(torch, run, seconds: float = 1.5):
    """Mean graphics clock (MHz) over the GPU's XCDs while `run` (one GEMM
    call) repeats back to back for about `seconds`, from amd-smi's metrics
    table.  The table refreshes with a lag of about half a second, so only
    samples from the second half of the loop, with the GPU fully busy, count.
    None where amd-smi is not available or no sample qualifies."""
    import threading
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        bus = torch.cuda.get_device_properties(0).pci_bus_id
        match = [h for h in handles if int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus]
        h = match[0] if len(match) == 1 else (handles[0] if len(handles) == 1 else None)
        if h is None:
            amdsmi.amdsmi_shut_down()
            return None
        amdsmi.amdsmi_get_gpu_metrics_info(h)
    except Exception:
        return None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        run()
    e1.record()
    torch.cuda.synchronize()
    calls = max(10, int(seconds / (e0.elapsed_time(e1) * 1e-3 / 5)))
    samples, done = [], threading.Event()

    def sample():
        while not done.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                clks = m.get("current_gfxclks")
                clks = [c for c in clks if isinstance(c, int)] if isinstance(clks, list) else []
                if not clks and isinstance(m.get("current_gfxclk"), int):
                    clks = [m["current_gfxclk"]]
                samples.append((time.perf_counter(), clks, m.get("average_gfx_activity")))
            except Exception:
                pass
            time.sleep(0.02)

    th = threading.Thread(target=sample, daemon=True)
    t0 = time.perf_counter()
    th.start()
    for _ in range(calls):
        run()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    done.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    mid = t0 + 0.5 * (t1 - t0)
    good = [c for t, clks, act in samples if t >= mid and isinstance(act, int) and act >= 90 for c in clks]
    return round(float(np.mean(good)), 1) if good else None


def calibrate_copy(mib: int):
    """A plain device-to-device copy of known size: read mib MiB, write mib MiB.
    Under rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE give the factor that
    turns those counters into bytes."""
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4}), flush=True)


class Step:
    """Device buffers and the callable that runs one step."""

    def __init__(self, workload: str, torch, fp8, synth):
        self.torch, self.fp8 = torch, fp8
        self.workload = workload
        dev = torch.device("cuda:0")
        self.dev = dev

        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

        if workload == "tiny":
            X, W = synth.tiny()
            xs, ws = [torch.from_numpy(X).to(dev)], [torch.from_numpy(W).to(dev)]
            self.M, self.N, self.K = 256, 256, 256
            self.in_bytes = 4
        elif workload in ("mlp8b", "qkv", "mlp70b"):
            X, W = getattr(synth, workload)()
            self.M, self.K = X.shape
            self.N = W.shape[0]
            x0, w0 = bf16(X), bf16(W)
            del X, W
            # rotate input copies so that no quantize input is still in the
            # 256 MB Infinity Cache from the previous step
            per = (x0.numel() + w0.numel()) * 2
            copies = max(1, min(4, -(-600 * 2 ** 20 // per)))
            xs = [x0] + [x0.clone() for _ in range(copies - 1)]
            ws = [w0] + [w0.clone() for _ in range(copies - 1)]
            self.in_bytes = 2
        elif workload == "moe":
            cfg = synth.CONFIGS["moe"]
            X, offsets, _ = synth.moe_routing(cfg["tokens"], cfg["top_k"], cfg["experts"], cfg["K"])
            self.M, self.K = X.shape
            self.N = cfg["N"]
            E = cfg["experts"]
            x0 = bf16(X)
            del X
            xs = [x0] + [x0.clone() for _ in range(3)]
            # expert weights: served in FP8, cast once outside the timed steps
            self.wq_e = torch.empty((E, self.N, self.K), dtype=torch.uint8, device=dev)
            self.sw_e = torch.empty(E, dtype=torch.float32, device=dev)
            for e in range(E):
                fp8.quantize(bf16(synth.moe_weight(e, self.N, self.K)), "e4m3", "tensor", out=self.wq_e[e],
                             scale_inv_out=self.sw_e[e:e + 1].view(1, 1))
            self.offs = torch.from_numpy(offsets.astype(np.int32)).to(dev)
            ws = [self.wq_e]
            self.in_bytes = 2
        elif workload == "dgrad":
            dy, w = synth.dgrad()
            self.M, self.K = dy.shape            # tokens, layer outputs (the reduction)
            self.N = w.shape[1]                  # layer inputs
            d0, w0 = bf16(dy), bf16(w)
            del dy, w
            per = (d0.numel() + w0.numel()) * 2
            copies = max(1, min(4, -(-600 * 2 ** 20 // per)))
            xs = [d0] + [d0.clone() for _ in range(copies - 1)]
            ws = [w0] + [w0.clone() for _ in range(copies - 1)]
            self.in_bytes = 2
            self.h_dy = fp8.AmaxHistory(16)
        else:  # wgrad
            dy, x = synth.wgrad_step(0)
            self.M = self.N = dy.shape[1]
            self.K = dy.shape[0]
            xs = [bf16(dy)] + [bf16(synth.wgrad_step(t)[0]) for t in (1, 2)]
            ws = [bf16(x)] + [bf16(synth.wgrad_step(t)[1]) for t in (1, 2)]
            self.in_bytes = 2
            self.h_dy, self.h_x = fp8.AmaxHistory(16), fp8.AmaxHistory(16)
        self.xs, self.ws = xs, ws
        self.i = 0
        M, N, K = self.M, self.N, self.K
        T = torch
        # outputs, allocated once
        if workload == "dgrad":
            self.xq = T.empty((M, K), dtype=T.uint8, device=dev)        # dY
            self.xqt = T.empty((K, M), dtype=T.uint8, device=dev)       # dY^T (the wgrad operand)
            self.wq = T.empty((N, K), dtype=T.uint8, device=dev)        # W^T
        elif workload == "wgrad":
            self.xq = T.empty((M, K), dtype=T.uint8, device=dev)
            self.wq = T.empty((N, K), dtype=T.uint8, device=dev)
        else:
            self.xq = T.empty((M, K), dtype=T.uint8, device=dev)
            self.wq = T.empty((N, K), dtype=T.uint8, device=dev)
        gx = {"tiny": "tensor", "mlp8b": "tensor", "qkv": "row", "mlp70b": "1x128", "wgrad": "tensor",
              "dgrad": "tensor", "moe": "row"}[workload]
        gw = {"tiny": "tensor", "mlp8b": "tensor", "qkv": "row", "mlp70b": "128x128", "wgrad": "tensor",
              "dgrad": "tensor", "moe": "tensor"}[workload]
        self.gx, self.gw = gx, gw
        rows_x, cols_x = xs[0].shape
        rows_w, cols_w = ws[0].shape[-2:]
        self.sx = T.empty(fp8.group_grid(gx, rows_x, cols_x), dtype=T.float32, device=dev)
        self.ax = T.empty_like(self.sx)
        self.sw = T.empty(fp8.group_grid(gw, rows_w, cols_w), dtype=T.float32, device=dev)
        self.aw = T.empty_like(self.sw)
        out_dt = T.float32 if workload in ("tiny", "wgrad") else T.bfloat16
        self.y = T.empty((M, N), dtype=out_dt, device=dev)
        self.elems = xs[0].numel() + (0 if workload == "moe" else ws[0].numel())

    def quantize(self, dx=None, dw=None):
        """Cast this step's operands; dx, dw: optional fp8.Diag counters of
        the first and the second operand's cast."""
        fp8, i = self.fp8, self.i
        x, w = self.xs[i % len(self.xs)], self.ws[i % len(self.ws)]
        self.last_inputs = (x, w)
        if self.workload == "dgrad":
            fp8.quantize_dual(x, "e5m2", history=self.h_dy, diag=dx, out=self.xq, out_t=self.xqt,
                              scale_inv_out=self.sx, amax_out=self.ax)
            fp8.quantize(w, "e4m3", "tensor", transpose=True, diag=dw, out=self.wq, scale_inv_out=self.sw,
                         amax_out=self.aw)
        elif self.workload == "wgrad":
            fp8.quantize(x, "e5m2", "tensor", history=self.h_dy, transpose=True, diag=dx, out=self.xq,
                         scale_inv_out=self.sx, amax_out=self.ax)
            fp8.quantize(w, "e4m3", "tensor", history=self.h_x, transpose=True, diag=dw, out=self.wq,
                         scale_inv_out=self.sw, amax_out=self.aw)
        elif self.workload == "moe":
            fp8.quantize(x, "e4m3", "row", diag=dx, out=self.xq, scale_inv_out=self.sx, amax_out=self.ax)
        elif self.gx == "tensor" and self.gw == "tensor":
            # both operands per tensor, just in time: one amax and one cast launch for the two
            fp8.quantize_tensors([x, w], "e4m3", outs=[self.xq, self.wq], diags=[dx, dw],
                                 scale_inv_outs=[self.sx, self.sw], amax_outs=[self.ax, self.aw])
        else:
            pow2 = self.workload == "qkv"
            fp8.quantize(x, "e4m3", self.gx, pow2=pow2, diag=dx, out=self.xq, scale_inv_out=self.sx,
                         amax_out=self.ax)
            fp8.quantize(w, "e4m3", self.gw, pow2=pow2, diag=dw, out=self.wq, scale_inv_out=self.sw,
                         amax_out=self.aw)

    def gemm(self):
        fp8 = self.fp8
        if self.workload == "mlp70b":
            fp8.blockscaled_gemm(self.xq, self.wq, self.sx, self.sw, out=self.y)
        elif self.workload == "moe":
            fp8.grouped_gemm(self.xq, self.wq_e, self.offs, self.sx.reshape(-1), self.sw_e, out=self.y)
        elif self.workload in ("wgrad", "dgrad"):
            fp8.scaled_gemm(self.xq, self.wq, self.sx.reshape(-1), self.sw.reshape(-1), "e5m2", "e4m3", out=self.y)
        else:
            fp8.scaled_gemm(self.xq, self.wq, self.sx.reshape(-1), self.sw.reshape(-1), out=self.y)
        self.i += 1

    def quant_errors(self, counts=None) -> dict:
        """Relative error of each operand's cast (the last quantize's inputs,
        codes and scales), with its saturation / non-finite / underflow
        counts when `counts` (the two fp8.Diag of that quantize) is given."""
        t, (x, w) = self.torch, self.last_inputs
        if self.workload == "wgrad":      # dY^T in E5M2, X^T in E4M3, per tensor
            ops = [("dY", x, self.xq, self.sx, "e5m2", "tensor", True),
                   ("X", w, self.wq, self.sw, "e4m3", "tensor", True)]
        elif self.workload == "dgrad":    # dY in E5M2 (delayed), W^T in E4M3
            ops = [("dY", x, self.xq, self.sx, "e5m2", "tensor", False),
                   ("W", w, self.wq, self.sw, "e4m3", "tensor", True)]
        else:
            ops = [("X", x, self.xq, self.sx, "e4m3", self.gx, False)]
            if self.workload != "moe":    # the experts' weights are cast once, outside the steps
                ops.append(("W", w, self.wq, self.sw, "e4m3", self.gw, False))
        out = {}
        for k, (name, a, q, s, f, g, tr) in enumerate(ops):
            out[name] = {"rel_err": round(quant_rel_err(t, a, q, s, f, g, tr), 6), "granularity": g, "format": f}
            if counts is not None:
                out[name].update(counts[k].read())
        return out

    def quant_bytes(self) -> float:
        """Algorithmic HBM bytes of the two casts of one step."""
        e = self.elems
        if self.workload in ("tiny", "mlp8b"):
            return e * (2 * self.in_bytes + 1)      # amax pass + cast pass
        if self.workload == "wgrad":
            return e * (self.in_bytes + 1)          # delayed: one pass
        if self.workload == "dgrad":
            nd, nw = self.M * self.K, self.N * self.K
            return nd * (self.in_bytes + 2) + nw * (2 * self.in_bytes + 1)   # dY delayed, 2 outputs; W two-pass
        return e * (self.in_bytes + 1)              # row / block: one pass (scales negligible)


class KvStep:
    """The KV-cache step: store K and V of the new chunk, gather the context."""

    LAYERS = 4     # rotated so that one step's caches are not left in the 256 MB Infinity Cache

    def __init__(self, torch, fp8, synth):
        cfg = synth.CONFIGS["kv"]
        self.H, self.D, self.cap, self.n = cfg["heads"], cfg["head_dim"], cfg["capacity"], cfg["new_tokens"]
        dev = torch.device("cuda:0")

        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

        pages = synth.kv_pages(self.cap, cfg["page"])
        self.pt = torch.from_numpy(pages).to(dev)
        self.new_slots = self.pt[self.cap - self.n:].contiguous()
        self.k = [bf16(synth.kv_keys(self.n, self.H, self.D, seed=11 + 100 * i)) for i in range(self.LAYERS)]
        self.v = [bf16(synth.kv_values(self.n, self.H, self.D, seed=12 + 100 * i)) for i in range(self.LAYERS)]
        self.cache = fp8.KVCache(self.LAYERS, self.cap, self.H, self.D, device=dev)
        old = bf16(synth.kv_values(self.cap - self.n, self.H, self.D, seed=21))
        old_slots = self.pt[:self.cap - self.n].contiguous()
        for layer in range(self.LAYERS):
            self.cache.store(layer, old, old, old_slots)
        self.ko = torch.empty((self.cap, self.H * self.D), dtype=torch.bfloat16, device=dev)
        self.vo = torch.empty_like(self.ko)
        self.fp8 = fp8
        self.i = 0

    def store(self):
        L = self.i % self.LAYERS
        self.cache.store(L, self.k[L], self.v[L], self.new_slots)

    def load(self):
        L = self.i % self.LAYERS
        self.cache.k[L].load(slots=self.pt, out=self.ko)
        self.cache.v[L].load(slots=self.pt, out=self.vo)
        self.i += 1

    def store_bytes(self) -> float:
        """Algorithmic HBM bytes of the two stores: bf16 in, codes and one
        fp32 scale per (token, head) out, the slot of each token read."""
        n, H, D = self.n, self.H, self.D
        return 2 * (n * H * D * (2 + 1) + n * H * 4 + n * 8)

    def load_bytes(self) -> float:
        """The two gathers: codes and scales in, bf16 out, a slot per row."""
        c, H, D = self.cap, self.H, self.D
        return 2 * (c * H * D * (1 + 2) + c * H * 4 + c * 8)


def kv_cpu_baseline(synth):
    """The oracle, untuned, on one whole KV step (one layer): store the 8192
    new tokens of K and V, gather all 32768 rows of each; GB/s by the same
    byte count.  Its loops run per (token, head) vector, one row at a time,
    so one core does the work."""
    import oracle
    cfg = synth.CONFIGS["kv"]
    H, D, cap = cfg["heads"], cfg["head_dim"], cfg["capacity"]
    n, m = cfg["new_tokens"], cap
    pages = synth.kv_pages(cap, cfg["page"])
    k = synth.kv_keys(n, H, D)
    v = synth.kv_values(n, H, D)
    ck = np.zeros((cap, H, D), np.uint8)
    cv = np.zeros((cap, H, D), np.uint8)
    sk = np.zeros((cap, H), np.float32)
    sv = np.zeros((cap, H), np.float32)
    t0 = time.perf_counter()
    oracle.kv_store(k, H, D, ck, sk, slots=pages[cap - n:])
    oracle.kv_store(v, H, D, cv, sv, slots=pages[cap - n:])
    oracle.kv_load(ck, sk, m, slots=pages[:m])
    oracle.kv_load(cv, sv, m, slots=pages[:m])
    dt = time.perf_counter() - t0
    nbytes = 2 * (n * H * D * 3 + n * H * 4 + n * 8) + 2 * (m * H * D * 3 + m * H * 4 + m * 8)
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "store %d tokens of K and V (8 heads x 128, E4M3 per token-head) through the page "
                      "table, gather %d rows of each to bf16: %.1f s" % (n, m, dt)}


def kv_main(args, torch, fp8, synth):
    st = KvStep(torch, fp8, synth)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        st.store()
        st.load()
    K = args.steps

    def step():
        st.store()
        st.load()

    def store_only():                 # advances the layer as a step does
        st.store()
        st.i += 1

    # the K steps timed as a whole, then each operation back to back
    ms = loop_ms(torch, step, K)
    s_ms = loop_ms(torch, store_only, K)
    l_ms = loop_ms(torch, st.load, K)
    sb, lb = st.store_bytes(), st.load_bytes()
    s_gbs, l_gbs = sb / (s_ms * 1e-3) / 1e9, lb / (l_ms * 1e-3) / 1e9
    # the gather kernel dominates; its launches are the two loads of a step
    per_launch = lb / 2
    tb, tnote = traffic("kv")
    roof = {"bound": "hbm", "achieved": round(l_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(l_gbs / PEAK_HBM_GBS, 4), "traffic": tb, "traffic_note": tnote,
            "algorithmic_bytes_per_launch": int(per_launch),
            "time": "load_ms: mean of K back-to-back gathers between two events, per launch"}
    cpu = None if args.no_cpu_baseline else kv_cpu_baseline(synth)
    out = {
        "metric": "FP8 KV-cache store + paged gather-dequantize GB/s (% HBM peak)",
        "value": round((sb + lb) / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 codes + fp32 scales (bf16 in/out)",
        "data": "synthetic (seeded numpy PCG64)",
        "config": {"workload": WORKLOADS["kv"], "heads": st.H, "head_dim": st.D, "capacity": st.cap,
                   "new_tokens": st.n},
        "kernels": {
            "store_ms": round(s_ms, 4), "store_gbs": round(s_gbs, 1),
            "load_ms": round(l_ms, 4), "load_gbs": round(l_gbs, 1),
            "store_bytes": int(sb), "load_bytes": int(lb),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


CONFIG_WORKLOADS = ("qkv", "mlp70b", "wgrad", "dgrad", "moe")


def workload_block(torch, fp8, synth, workload: str, steps: int) -> dict:
    """One other GEMM workload timed in the same run, so that one default
    bench line records every configuration: whole steps, its GEMM (the mean
    over `steps` steps of the call between two events around it), its
    quantize (calls back to back between two events), with the GEMM's
    TFLOP/s and fraction of the FP8 MFMA peak."""
    st = Step(workload, torch, fp8, synth)
    for _ in range(3):
        st.quantize()
        st.gemm()

    def step():
        st.quantize()
        st.gemm()

    def quantize_only():
        st.quantize()
        st.i += 1

    with phase(torch, "workload %s" % workload):
        ms = loop_ms(torch, step, steps)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e in ev:
            st.quantize()
            e[0].record()
            st.gemm()
            e[1].record()
        torch.cuda.synchronize()
        g_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        q_ms = loop_ms(torch, quantize_only, steps)
    flops = 2.0 * st.M * st.N * st.K
    tflops = flops / (g_ms * 1e-3) / 1e12
    qbytes = st.quant_bytes()
    out = {"M": st.M, "N": st.N, "K": st.K, "steps": steps,
           "gemm_ms": round(g_ms, 4), "gemm_tflops": round(tflops, 2),
           "gemm_frac_fp8_peak": round(tflops / PEAK_FP8_TFLOPS, 4),
           "quantize_ms": round(q_ms, 4), "quantize_gbs": round(qbytes / (q_ms * 1e-3) / 1e9, 1),
           "quantize_frac_hbm_peak": round(qbytes / (q_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "step_ms": round(ms, 4), "step_tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
    del st
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, workload, synth):
    """The oracle, untuned, on a bounded sample of the same step: quantize the
    first `cpu_rows` rows of X and `cpu_cols` rows of W (half as many of
    each for the block-scaled workload, whose K is twice as long), then the
    GEMM block Y[:cpu_rows, :cpu_cols] with the full K, on all the threads
    it gets; the quantize again on one thread.  `value` is the sample's
    whole-step rate; the quantize (algorithmic bytes, as on the GPU) and the
    GEMM are also reported on their own.  The backward workloads take the
    GEMM operands as the GPU casts them (transposed slices, E5M2 gradients);
    the grouped one takes routed rows of one expert with that expert's
    weight, cast outside the step as on the GPU."""
    import oracle
    if workload not in ("mlp8b", "tiny", "qkv", "mlp70b", "wgrad", "dgrad", "moe"):
        return None
    gx = gw = "tensor"
    fx, fw = oracle.E4M3, oracle.E4M3
    pow2 = block = False
    w_in_step = True                     # the weight's cast is part of the step
    if workload == "tiny":
        X, W = synth.tiny()
        r, c = 256, 256
    elif workload in ("wgrad", "dgrad"):
        # the GEMM operands as the GPU casts them: dW = (dY^T)(X^T)^T over the
        # tokens, dX = dY (W^T)^T over the layer's outputs; E5M2 gradients
        fx = oracle.E5M2
        if workload == "wgrad":
            dy, x = synth.wgrad_step(0)
            r, c = args.cpu_rows // 2, args.cpu_cols // 2
            X, W = np.ascontiguousarray(dy[:, :r].T), np.ascontiguousarray(x[:, :c].T)
        else:
            dy, w = synth.dgrad()
            r, c = args.cpu_rows // 4, args.cpu_cols // 2
            X, W = np.ascontiguousarray(dy[:r]), np.ascontiguousarray(w[:, :c].T)
    elif workload == "moe":
        # the first routed rows, all in expert 0's group, times that expert's
        # weight (served in FP8: cast once, outside the step, as on the GPU)
        cfg = synth.CONFIGS["moe"]
        Xr, offsets, _ = synth.moe_routing(cfg["tokens"], cfg["top_k"], cfg["experts"], cfg["K"])
        r, c = min(args.cpu_rows, int(offsets[1] - offsets[0])), args.cpu_cols
        X = np.ascontiguousarray(Xr[int(offsets[0]):int(offsets[0]) + r])
        W = np.ascontiguousarray(synth.moe_weight(0, cfg["N"], cfg["K"])[:c])
        gx, w_in_step = "row", False
    else:
        r, c = args.cpu_rows, args.cpu_cols
        if workload == "qkv":
            gx = gw = "row"
            pow2 = True
        elif workload == "mlp70b":      # K = 8192: half the rows and columns keep the sample's time alike
            gx, gw, block = "1x128", "128x128", True
            r, c = r // 2, c // 2
        X, W = getattr(synth, workload)()
        X, W = np.ascontiguousarray(X[:r]), np.ascontiguousarray(W[:c])
    r, c = X.shape[0], W.shape[0]        # a sample past a tensor's end takes all of it
    K = X.shape[1]
    in_bytes = X.dtype.itemsize          # bf16 bits (uint16) or fp32
    # the GPU's algorithmic bytes: a just-in-time per-tensor cast reads its
    # input twice (the delayed casts of the backward workloads once)
    passes = 2 if gx == "tensor" and workload not in ("wgrad", "dgrad") else 1
    qbytes = (X.size + (W.size if w_in_step else 0)) * (passes * in_bytes + 1)
    qw_fixed = None if w_in_step else oracle.quantize(W, fw, gw, pow2=pow2)

    def quantize_both():
        qx = oracle.quantize(X, fx, gx, pow2=pow2)
        return qx, (oracle.quantize(W, fw, gw, pow2=pow2) if w_in_step else qw_fixed)

    t0 = time.perf_counter()
    qx, qw = quantize_both()
    t1 = time.perf_counter()
    if block:
        ms, ns = np.repeat(np.arange(r), c), np.tile(np.arange(c), r)
        oracle.blockgemm_sampled(qx["q"], qw["q"], qx["scale_inv"], qw["scale_inv"], ms, ns)
    else:
        oracle.gemm(qx["q"], fx, qw["q"], fw, qx["scale_inv"].reshape(-1), qw["scale_inv"].reshape(-1), with_p=True)
    t2 = time.perf_counter()
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        t3 = time.perf_counter()
        quantize_both()
        t4 = time.perf_counter()
    finally:
        oracle.set_num_threads(threads)
    dt = t2 - t0
    what = {"tensor": "per-tensor E4M3", "row": "per-row power-of-two E4M3",
            "1x128": "E4M3, X in 1x128 and W in 128x128 blocks"}[gx]
    if workload == "wgrad":
        sample = ("quantize dY[:, :%d]^T (E5M2), X[:, :%d]^T (E4M3), per tensor + GEMM dW[:%d, :%d] with K=%d "
                  "tokens: %.1f s" % (r, c, r, c, K, dt))
    elif workload == "dgrad":
        sample = ("quantize dY[:%d] (E5M2), W[:, :%d]^T (E4M3), per tensor + GEMM dX[:%d, :%d] with K=%d: %.1f s"
                  % (r, c, r, c, K, dt))
    elif workload == "moe":
        sample = ("quantize %d routed rows of expert 0 (per-row E4M3) + GEMM with its FP8 weight W_0[:%d] "
                  "(cast outside the step) with K=%d: %.1f s" % (r, c, K, dt))
    else:
        sample = "quantize X[:%d], W[:%d] (%s) + GEMM Y[:%d, :%d] with K=%d: %.1f s" % (r, c, what, r, c, K, dt)
    return {"value": 2.0 * r * c * K / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": sample,
            "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)),
            "quantize_gbs": round(qbytes / (t1 - t0) / 1e9, 3),
            "quantize_gbs_1_thread": round(qbytes / (t4 - t3) / 1e9, 3),
            "gemm_gflops": round(2.0 * r * c * K / (t2 - t1) / 1e9, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    import torch
    import fp8_precision_quantization_amd as fp8
    import synth

    if args.workload == "kv":
        kv_main(args, torch, fp8, synth)
        return
    st = Step(args.workload, torch, fp8, synth)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        st.quantize()
        st.gemm()
    K = args.steps

    def step():
        st.quantize()
        st.gemm()

    def quantize_only():              # advances the input rotation as a step does
        st.quantize()
        st.i += 1

    # the K steps, timed as a whole: only the work between the two events
    with phase(torch, "timed steps"):
        ms = loop_ms(torch, step, K)
    # K more steps with events around each operation: each launch's duration
    # as it runs in a step (these include the events' own short gaps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    with phase(torch, "steps with events"):
        for s in range(K):
            ev[s][0].record()
            st.quantize()
            ev[s][1].record()
            st.gemm()
            ev[s][2].record()
        torch.cuda.synchronize()
    q_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])
    g_ms = np.array([b.elapsed_time(c) for _, b, c in ev])
    g_step = float(g_ms.mean())
    # each operation on its own, back to back: a GEMM then also absorbs the
    # write-back of the previous one's output, which in a step the quantize does
    with phase(torch, "gemm back to back"):
        g_b2b = loop_ms(torch, st.gemm, K)
    with phase(torch, "quantize back to back"):
        q_mean = loop_ms(torch, quantize_only, K)
    flops = 2.0 * st.M * st.N * st.K
    gemm_tflops = flops / (g_step * 1e-3) / 1e12
    qbytes = st.quant_bytes()
    q_gbs = qbytes / (q_mean * 1e-3) / 1e9
    # after the timed region: the streaming probes' ceilings (before the
    # clock probe's 1.5 s of GEMMs heat the chip), and the graphics clock
    # under the GEMM
    with phase(torch, "stream ceilings"):
        ceil = stream_ceilings(torch)
    with phase(torch, "clock under the gemm"):
        clock = None if args.no_clock else gemm_clock_mhz(torch, st.gemm)
    diags = (fp8.Diag(), fp8.Diag())
    st.quantize(*diags)
    q_err = st.quant_errors(diags)
    others = None
    if not args.no_configs:
        others = {}
        for w in CONFIG_WORKLOADS:
            if w != args.workload:
                others[w] = workload_block(torch, fp8, synth, w, args.config_steps)
    tb, tnote = traffic(args.workload)
    roof = {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "traffic": tb, "traffic_note": tnote,
            "time": "kernels.gemm_ms: mean over K steps of the GEMM call between two events around it"}
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, args.workload, synth)
    out = {
        "metric": "FP8 scaled-GEMM TFLOPS (% of FP8 MFMA peak); quantize GB/s (% HBM peak)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (e4m3/e5m2 operands, fp32 accumulate)",
        "data": "synthetic (seeded numpy PCG64)",
        "config": {"workload": WORKLOADS[args.workload], "M": st.M, "N": st.N, "K": st.K},
        "kernels": {
            "gemm_ms": round(g_step, 4),
            "gemm_tflops": round(gemm_tflops, 2),
            "gemm_pct_fp8_peak": round(100 * gemm_tflops / PEAK_FP8_TFLOPS, 2),
            "gemm_ms_spread": spread(g_ms),
            "gemm_ms_back_to_back": round(g_b2b, 4),
            "gemm_tflops_back_to_back": round(flops / (g_b2b * 1e-3) / 1e12, 2),
            "gemm_clock_mhz": clock,
            "gemm_pct_fp8_peak_at_clock": (round(100 * gemm_tflops / (PEAK_FP8_TFLOPS * clock / 2400.0), 2)
                                           if clock else None),
            "quantize_ms": round(q_mean, 4),
            "quantize_ms_spread": spread(q_ms),
            # the quantize's share of a step (step minus the GEMM): it also
            # pays for writing back the previous GEMM's cached output
            "quantize_ms_in_step": round(ms - g_step, 4),
            "quantize_gbs_in_step": round(qbytes / ((ms - g_step) * 1e-3) / 1e9, 1) if ms > g_step else None,
            "quantize_gbs": round(q_gbs, 1),
            "quantize_pct_hbm_peak": round(100 * q_gbs / PEAK_HBM_GBS, 2),
            "quantize_bytes": int(qbytes),
            "quantize_rel_err": q_err,
            "stream_ceilings": ceil,
            # against the probe with the cast's own 2:1 read:write pattern
            "quantize_pct_read2_write1_ceiling": round(100 * q_gbs / ceil["read2_write1_gbs"], 2),
            # the other GEMM workloads, each timed in this run (GEMM, quantize
            # and whole steps; TFLOP/s and fraction of the FP8 peak)
            "workloads": others,
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
