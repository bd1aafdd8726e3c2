"""FP8 scaled quantization and scaled FP8 GEMM for AMD MI355X (gfx950).

Thin Python binding over the C ABI in include/fp8mi.h (libfp8mi.so).  torch
tensors serve only as device memory and streams: every step of the
computation runs in the library's HIP kernels.  There is no CPU path; every
call raises if the library is missing or the device is not gfx950.

    import fp8_precision_quantization_amd as fp8
    xq = fp8.quantize(x, "e4m3", "tensor")          # x: bf16/fp32 [rows, cols] on cuda
    wq = fp8.quantize(w, "e4m3", "tensor")
    y = fp8.scaled_gemm(xq.q, wq.q, xq.scale_inv, wq.scale_inv)   # y = x w^T, bf16
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import Fp8Error  # noqa: F401

__all__ = ["quantize", "quantize_dual", "quantize_tensors", "amax", "scaled_gemm", "blockscaled_gemm", "AmaxHistory", "Diag",
           "QuantResult", "Fp8Error", "FORMATS", "GRANULARITIES", "group_grid", "kv_store", "kv_load",
           "KVTensorCache", "KVCache", "grouped_gemm", "workspace"]

FORMATS = {"e4m3": _lib.FP8_E4M3, "e5m2": _lib.FP8_E5M2}
GRANULARITIES = {"tensor": _lib.FP8_GRAN_TENSOR, "row": _lib.FP8_GRAN_ROW,
                 "1x128": _lib.FP8_GRAN_BLOCK_1x128, "128x128": _lib.FP8_GRAN_BLOCK_128x128}
TORCH_FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def _fmt(f) -> int:
    if isinstance(f, str):
        return FORMATS[f]
    return int(f)


def _gran(g) -> int:
    if isinstance(g, str):
        return GRANULARITIES[g]
    return int(g)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _same_device(t: torch.Tensor, device: torch.device, name: str) -> None:
    if t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))


def _matrix(x: torch.Tensor, name: str):
    if x.dim() != 2:
        raise ValueError("%s must be 2-D, got shape %s" % (name, tuple(x.shape)))
    if not x.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if x.stride(1) != 1 and x.shape[1] > 1:
        raise ValueError("%s must have a contiguous last dimension" % name)
    return x.shape[0], x.shape[1], max(x.stride(0), 1) if x.shape[0] > 1 else max(x.shape[1], 1)


def _buf(t: torch.Tensor, n: int, dtype, device: torch.device, name: str) -> int:
    """Pointer of a buffer the library reads or writes as n packed elements
    of dtype on device; raises before any launch if t is not one."""
    if not isinstance(t, torch.Tensor) or t.device != device:
        raise ValueError("%s must be a tensor on %s" % (name, device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.numel() != n or not t.is_contiguous():
        raise ValueError("%s must be a contiguous tensor of %d elements, got shape %s"
                         % (name, n, tuple(t.shape)))
    return t.data_ptr()


def _out_matrix(out: torch.Tensor, rows: int, cols: int, dtype, device: torch.device, name: str) -> int:
    """Leading dimension of an output matrix [rows, cols] of dtype on device
    with a contiguous last dimension; raises before any launch if out is not one."""
    if not isinstance(out, torch.Tensor) or out.device != device:
        raise ValueError("%s must be a tensor on %s" % (name, device))
    if out.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, out.dtype))
    if tuple(out.shape) != (rows, cols):
        raise ValueError("%s must have shape %s, got %s" % (name, (rows, cols), tuple(out.shape)))
    if cols > 1 and out.stride(1) != 1:
        raise ValueError("%s must have a contiguous last dimension" % name)
    return max(out.stride(0), 1) if rows > 1 else max(cols, 1)


def workspace(device="cuda") -> torch.Tensor:
    """A workspace for the calls that need one (fp8_workspace_size() bytes).
    Calls ordered on one stream may share it; calls running concurrently on
    different streams need one each."""
    return torch.empty(_lib.WORKSPACE_BYTES, dtype=torch.uint8, device=device)


def _workspace(ws: Optional[torch.Tensor], needed: bool, device: torch.device):
    """(tensor kept alive for the call, pointer, bytes).  Without one given, a
    needed workspace comes from torch's allocator, whose blocks are reused in
    the order of the current stream."""
    if not needed and ws is None:
        return None, None, 0
    if ws is None:
        ws = workspace(device)
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % device)
    nbytes = ws.numel() * ws.element_size()
    if nbytes < _lib.WORKSPACE_BYTES:
        raise ValueError("workspace must hold %d bytes, got %d" % (_lib.WORKSPACE_BYTES, nbytes))
    return ws, ws.data_ptr(), nbytes


def _numel(shape) -> int:
    n = 1
    for d in shape:
        n *= d
    return n


def group_grid(granularity, rows: int, cols: int):
    g = _gran(granularity)
    if g == _lib.FP8_GRAN_TENSOR:
        return (1,)
    if g == _lib.FP8_GRAN_ROW:
        return (rows,)
    if g == _lib.FP8_GRAN_BLOCK_1x128:
        return (rows, (cols + 127) // 128)
    return ((rows + 127) // 128, (cols + 127) // 128)


class Diag:
    """Device counters (sat, nonfinite, underflow); the library adds to them."""

    def __init__(self, device="cuda"):
        self.buf = torch.zeros(4, dtype=torch.int32, device=device)

    def zero_(self):
        self.buf.zero_()
        return self

    def read(self) -> dict:
        v = self.buf.cpu().tolist()
        return {"sat": v[0], "nonfinite": v[1], "underflow": v[2]}


class AmaxHistory:
    """Delayed-scaling state: a 128-byte device struct (fp8_amax_history)."""

    def __init__(self, length: int = 16, device="cuda"):
        self.buf = torch.empty(_lib.HISTORY_BYTES // 4, dtype=torch.int32, device=device)
        self.length = length
        self.reset()

    def reset(self):
        dev = self.buf.device
        _lib.check(_lib.lib().fp8_history_init(self.buf.data_ptr(), self.length, _stream(dev)),
                   "fp8_history_init")

    def set_guard(self, threshold: float):
        """Spike threshold for quantize(..., spike_guard=True); <= 0 is off."""
        dev = self.buf.device
        _lib.check(_lib.lib().fp8_history_set_guard(self.buf.data_ptr(), float(threshold), _stream(dev)),
                   "fp8_history_set_guard")

    def state(self) -> dict:
        w = self.buf.cpu()
        f = w.view(torch.float32)
        return {"amax": f[:16].clone(), "len": int(w[16]), "pos": int(w[17]), "count": int(w[18]),
                "scale": float(f[21]), "scale_inv": float(f[22]), "steps": int(w[23]),
                "spike_threshold": float(f[24]), "spikes": int(w[25]), "last_spiked": int(w[19])}

    def save(self) -> torch.Tensor:
        return self.buf.clone()

    def load(self, saved: torch.Tensor):
        self.buf.copy_(saved)


@dataclass
class QuantResult:
    q: torch.Tensor            # uint8 codes
    scale_inv: torch.Tensor    # fp32, group grid
    amax: torch.Tensor         # fp32, group grid
    fmt: str

    def as_float8(self) -> torch.Tensor:
        return self.q.view(TORCH_FP8[self.fmt])


def quantize(x: torch.Tensor, fmt="e4m3", granularity="tensor", pow2: bool = False,
             history: Optional[AmaxHistory] = None, transpose: bool = False,
             diag: Optional[Diag] = None, out: Optional[torch.Tensor] = None,
             spike_guard: bool = False,
             scale_inv_out: Optional[torch.Tensor] = None,
             amax_out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None) -> QuantResult:
    rows, cols, ld = _matrix(x, "x")
    if x.dtype == torch.bfloat16:
        in_dt = _lib.FP8_IN_BF16
    elif x.dtype == torch.float32:
        in_dt = _lib.FP8_IN_F32
    else:
        raise TypeError("x must be bfloat16 or float32, got %s" % x.dtype)
    fmt_name = fmt if isinstance(fmt, str) else ("e4m3" if fmt == 0 else "e5m2")
    grid = group_grid(granularity, rows, cols)
    dev = x.device
    oshape = (cols, rows) if transpose else (rows, cols)
    if out is None:
        out = torch.empty(oshape, dtype=torch.uint8, device=dev)
    ldq = _out_matrix(out, oshape[0], oshape[1], torch.uint8, dev, "out")
    if scale_inv_out is None:
        scale_inv_out = torch.empty(grid, dtype=torch.float32, device=dev)
    if amax_out is None:
        amax_out = torch.empty(grid, dtype=torch.float32, device=dev)
    _buf(scale_inv_out, _numel(grid), torch.float32, dev, "scale_inv_out")
    _buf(amax_out, _numel(grid), torch.float32, dev, "amax_out")
    flags = ((_lib.FP8_SCALE_POW2 if pow2 else 0) | (_lib.FP8_TRANSPOSE_OUT if transpose else 0)
             | (_lib.FP8_SPIKE_GUARD if spike_guard else 0))
    ws, ws_ptr, ws_bytes = _workspace(workspace, _gran(granularity) == _lib.FP8_GRAN_TENSOR, dev)
    st = _lib.lib().fp8_quantize(
        x.data_ptr(), in_dt, rows, cols, ld, _fmt(fmt), _gran(granularity), flags,
        _ptr(history.buf) if history is not None else None, out.data_ptr(), ldq,
        scale_inv_out.data_ptr(), amax_out.data_ptr(), _ptr(diag.buf) if diag is not None else None,
        ws_ptr, ws_bytes, _stream(dev))
    _lib.check(st, "fp8_quantize")
    return QuantResult(out, scale_inv_out, amax_out, fmt_name)


def quantize_dual(x: torch.Tensor, fmt="e5m2", pow2: bool = False, history: Optional[AmaxHistory] = None,
                  diag: Optional[Diag] = None, spike_guard: bool = False,
                  out: Optional[torch.Tensor] = None, out_t: Optional[torch.Tensor] = None,
                  scale_inv_out: Optional[torch.Tensor] = None,
                  amax_out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None):
    """Per-tensor quantization into both layouts from one pass over x
    (fp8_quantize_dual).  Returns (QuantResult with q [rows x cols], qt [cols x rows])."""
    rows, cols, ld = _matrix(x, "x")
    if x.dtype == torch.bfloat16:
        in_dt = _lib.FP8_IN_BF16
    elif x.dtype == torch.float32:
        in_dt = _lib.FP8_IN_F32
    else:
        raise TypeError("x must be bfloat16 or float32, got %s" % x.dtype)
    fmt_name = fmt if isinstance(fmt, str) else ("e4m3" if fmt == 0 else "e5m2")
    dev = x.device
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if out_t is None:
        out_t = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    ldq = _out_matrix(out, rows, cols, torch.uint8, dev, "out")
    ldqt = _out_matrix(out_t, cols, rows, torch.uint8, dev, "out_t")
    if scale_inv_out is None:
        scale_inv_out = torch.empty((1, 1), dtype=torch.float32, device=dev)
    if amax_out is None:
        amax_out = torch.empty((1, 1), dtype=torch.float32, device=dev)
    _buf(scale_inv_out, 1, torch.float32, dev, "scale_inv_out")
    _buf(amax_out, 1, torch.float32, dev, "amax_out")
    flags = (_lib.FP8_SCALE_POW2 if pow2 else 0) | (_lib.FP8_SPIKE_GUARD if spike_guard else 0)
    ws, ws_ptr, ws_bytes = _workspace(workspace, True, dev)
    st = _lib.lib().fp8_quantize_dual(
        x.data_ptr(), in_dt, rows, cols, ld, _fmt(fmt), flags,
        _ptr(history.buf) if history is not None else None, out.data_ptr(), ldq, out_t.data_ptr(), ldqt,
        scale_inv_out.data_ptr(), amax_out.data_ptr(), _ptr(diag.buf) if diag is not None else None,
        ws_ptr, ws_bytes, _stream(dev))
    _lib.check(st, "fp8_quantize_dual")
    return QuantResult(out, scale_inv_out, amax_out, fmt_name), out_t


def quantize_tensors(xs, fmt="e4m3", pow2: bool = False, outs=None, diags=None, scale_inv_outs=None,
                     amax_outs=None, workspace: Optional[torch.Tensor] = None) -> list:
    """Just-in-time per-tensor quantization of up to 8 contiguous tensors in
    one amax launch and one cast launch (fp8_quantize_tensors).  xs: 2-D
    contiguous tensors of one dtype (bfloat16 or float32) on one device;
    outs: optional uint8 tensors of the same shapes; diags: optional Diag per
    tensor (None entries skip the counting); scale_inv_outs, amax_outs:
    optional one-element fp32 tensors per tensor.  Returns one QuantResult
    per tensor, each equal to quantize(x, fmt, "tensor", pow2)."""
    xs = list(xs)
    n = len(xs)
    if not 1 <= n <= _lib.MAX_TENSORS:
        raise ValueError("quantize_tensors takes 1..%d tensors, got %d" % (_lib.MAX_TENSORS, n))
    dev = xs[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must be device tensors, got %s" % dev)
    dt = xs[0].dtype
    if dt == torch.bfloat16:
        in_dt = _lib.FP8_IN_BF16
    elif dt == torch.float32:
        in_dt = _lib.FP8_IN_F32
    else:
        raise TypeError("tensors must be bfloat16 or float32, got %s" % dt)
    fmt_name = fmt if isinstance(fmt, str) else ("e4m3" if fmt == 0 else "e5m2")
    outs = list(outs) if outs is not None else [None] * n
    diags = list(diags) if diags is not None else [None] * n
    sinvs = list(scale_inv_outs) if scale_inv_outs is not None else [None] * n
    amaxs = list(amax_outs) if amax_outs is not None else [None] * n
    if len(outs) != n or len(diags) != n or len(sinvs) != n or len(amaxs) != n:
        raise ValueError("outs, diags, scale_inv_outs and amax_outs must have one entry per tensor")
    descs = (_lib.Fp8Tensor * n)()
    results = []
    for i, x in enumerate(xs):
        if x.dtype != dt:
            raise TypeError("tensor %d is %s, tensor 0 is %s" % (i, x.dtype, dt))
        _same_device(x, dev, "tensor %d" % i)
        if x.dim() != 2:
            raise ValueError("tensor %d must be 2-D, got shape %s" % (i, tuple(x.shape)))
        rows, cols = x.shape
        if x.numel() > 0 and not x.is_contiguous():
            raise ValueError("tensor %d must be contiguous" % i)
        out = outs[i]
        if out is None:
            out = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        _out_matrix(out, rows, cols, torch.uint8, dev, "outs[%d]" % i)
        if not out.is_contiguous():
            raise ValueError("outs[%d] must be contiguous" % i)
        sinv = sinvs[i] if sinvs[i] is not None else torch.empty((1, 1), dtype=torch.float32, device=dev)
        am = amaxs[i] if amaxs[i] is not None else torch.empty((1, 1), dtype=torch.float32, device=dev)
        _buf(sinv, 1, torch.float32, dev, "scale_inv_outs[%d]" % i)
        _buf(am, 1, torch.float32, dev, "amax_outs[%d]" % i)
        descs[i] = _lib.Fp8Tensor(x.data_ptr(), rows, cols, out.data_ptr(), sinv.data_ptr(), am.data_ptr(),
                                  _ptr(diags[i].buf) if diags[i] is not None else None)
        results.append(QuantResult(out, sinv, am, fmt_name))
    ws, ws_ptr, ws_bytes = _workspace(workspace, True, dev)
    st = _lib.lib().fp8_quantize_tensors(ctypes.cast(descs, ctypes.c_void_p), n, in_dt, _fmt(fmt), _lib.FP8_SCALE_POW2 if pow2 else 0,
                                         ws_ptr, ws_bytes, _stream(dev))
    _lib.check(st, "fp8_quantize_tensors")
    return results


def amax(x: torch.Tensor, granularity="tensor", out: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    rows, cols, ld = _matrix(x, "x")
    in_dt = _lib.FP8_IN_BF16 if x.dtype == torch.bfloat16 else _lib.FP8_IN_F32
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("x must be bfloat16 or float32")
    grid = group_grid(granularity, rows, cols)
    if out is None:
        out = torch.empty(grid, dtype=torch.float32, device=x.device)
    _buf(out, _numel(grid), torch.float32, x.device, "out")
    ws, ws_ptr, ws_bytes = _workspace(workspace, _gran(granularity) == _lib.FP8_GRAN_TENSOR, x.device)
    st = _lib.lib().fp8_amax(x.data_ptr(), in_dt, rows, cols, ld, _gran(granularity), out.data_ptr(),
                             ws_ptr, ws_bytes, _stream(x.device))
    _lib.check(st, "fp8_amax")
    return out


def _out_dtype(dt) -> int:
    if dt == torch.bfloat16:
        return _lib.FP8_OUT_BF16
    if dt == torch.float32:
        return _lib.FP8_OUT_F32
    raise TypeError("out dtype must be bfloat16 or float32")


def scaled_gemm(a_q: torch.Tensor, b_q: torch.Tensor, a_scale_inv: torch.Tensor,
                b_scale_inv: torch.Tensor, fa="e4m3", fb="e4m3", out_dtype=torch.bfloat16,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = (A_q . B_q^T) * sa * sb with A_q [M, K], B_q [N, K] uint8 codes."""
    M, K, lda = _matrix(a_q, "a_q")
    N, K2, ldb = _matrix(b_q, "b_q")
    if K != K2:
        raise ValueError("K mismatch: %d vs %d" % (K, K2))
    dev = a_q.device
    _same_device(b_q, dev, "b_q")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    ldc = _out_matrix(out, M, N, out.dtype, dev, "out")
    a_row = 0 if a_scale_inv.numel() == 1 else 1
    b_row = 0 if b_scale_inv.numel() == 1 else 1
    if a_row and a_scale_inv.numel() != M:
        raise ValueError("a_scale_inv must hold 1 or M=%d values" % M)
    if b_row and b_scale_inv.numel() != N:
        raise ValueError("b_scale_inv must hold 1 or N=%d values" % N)
    _buf(a_scale_inv, M if a_row else 1, torch.float32, dev, "a_scale_inv")
    _buf(b_scale_inv, N if b_row else 1, torch.float32, dev, "b_scale_inv")
    st = _lib.lib().fp8_scaled_gemm(a_q.data_ptr(), _fmt(fa), lda, b_q.data_ptr(), _fmt(fb), ldb, M, N, K,
                                    a_scale_inv.data_ptr(), a_row, b_scale_inv.data_ptr(), b_row,
                                    out.data_ptr(), _out_dtype(out.dtype), ldc, _stream(a_q.device))
    _lib.check(st, "fp8_scaled_gemm")
    return out


def blockscaled_gemm(a_q: torch.Tensor, b_q: torch.Tensor, a_scale_inv: torch.Tensor,
                     b_scale_inv: torch.Tensor, out_dtype=torch.bfloat16,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """E4M3 block-scaled GEMM: a_scale_inv [M, K/128], b_scale_inv [N/128, K/128]."""
    M, K, lda = _matrix(a_q, "a_q")
    N, K2, ldb = _matrix(b_q, "b_q")
    if K != K2:
        raise ValueError("K mismatch: %d vs %d" % (K, K2))
    dev = a_q.device
    _same_device(b_q, dev, "b_q")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    ldc = _out_matrix(out, M, N, out.dtype, dev, "out")
    if K % 128 == 0 and N % 128 == 0:     # else the library reports the unsupported shape
        _buf(a_scale_inv, M * (K // 128), torch.float32, dev, "a_scale_inv")
        _buf(b_scale_inv, (N // 128) * (K // 128), torch.float32, dev, "b_scale_inv")
    st = _lib.lib().fp8_blockscaled_gemm(a_q.data_ptr(), lda, b_q.data_ptr(), ldb, M, N, K,
                                         a_scale_inv.data_ptr(), b_scale_inv.data_ptr(), out.data_ptr(),
                                         _out_dtype(out.dtype), ldc, _stream(a_q.device))
    _lib.check(st, "fp8_blockscaled_gemm")
    return out


# ------------------------------------------------------------ grouped GEMM --
def grouped_gemm(a_q: torch.Tensor, b_q: torch.Tensor, group_offsets: torch.Tensor, a_scale_inv: torch.Tensor,
                 b_scale_inv: torch.Tensor, fa="e4m3", fb="e4m3", out_dtype=torch.bfloat16,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MoE grouped GEMM: rows [offs[g], offs[g+1]) of a_q [M, K] times expert
    g's b_q[g] ([G, N, K] uint8 codes): C[m] = (A_q[m] . B_q[g]^T) * sa * sb_g.
    group_offsets: int32 device tensor [G+1]; a_scale_inv: 1 or M values;
    b_scale_inv: G (one per expert) or G*N values.  Rows in no group are not
    written (out is allocated uninitialized when not given)."""
    M, K, lda = _matrix(a_q, "a_q")
    if b_q.dim() != 3 or not b_q.is_cuda or b_q.stride(2) != 1:
        raise ValueError("b_q must be a [G, N, K] device tensor with contiguous rows")
    G, N, K2 = b_q.shape
    if K != K2:
        raise ValueError("K mismatch: %d vs %d" % (K, K2))
    if (group_offsets.dtype != torch.int32 or not group_offsets.is_cuda or group_offsets.numel() != G + 1
            or not group_offsets.is_contiguous()):
        raise ValueError("group_offsets must be a contiguous int32 device tensor of G+1=%d entries" % (G + 1))
    ldb = b_q.stride(1) if N > 1 else K
    gstride = b_q.stride(0) if G > 1 else N * ldb
    dev = a_q.device
    _same_device(b_q, dev, "b_q")
    _same_device(group_offsets, dev, "group_offsets")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    ldc = _out_matrix(out, M, N, out.dtype, dev, "out")
    a_row = 0 if a_scale_inv.numel() == 1 else 1
    if a_row and a_scale_inv.numel() != M:
        raise ValueError("a_scale_inv must hold 1 or M=%d values" % M)
    if b_scale_inv.numel() == G:
        b_row = 0
    elif b_scale_inv.numel() == G * N:
        b_row = 1
    else:
        raise ValueError("b_scale_inv must hold G=%d or G*N=%d values" % (G, G * N))
    _buf(a_scale_inv, M if a_row else 1, torch.float32, dev, "a_scale_inv")
    _buf(b_scale_inv, G * N if b_row else G, torch.float32, dev, "b_scale_inv")
    ws, ws_ptr, ws_bytes = _workspace(workspace, True, dev)
    st = _lib.lib().fp8_grouped_gemm(a_q.data_ptr(), _fmt(fa), lda, b_q.data_ptr(), _fmt(fb), ldb, gstride, M, N, K,
                                     G, group_offsets.data_ptr(), a_scale_inv.data_ptr(), a_row,
                                     b_scale_inv.data_ptr(), b_row, out.data_ptr(), _out_dtype(out.dtype), ldc,
                                     ws_ptr, ws_bytes, _stream(a_q.device))
    _lib.check(st, "fp8_grouped_gemm")
    return out


# ------------------------------------------------------------ FP8 KV cache --
KV_STORAGE = {"e4m3": _lib.FP8_KV_E4M3, "e5m2": _lib.FP8_KV_E5M2, "bf16": _lib.FP8_KV_BF16}
KV_SCALING = {"token_head": _lib.FP8_KV_PER_TOKEN_HEAD, "head": _lib.FP8_KV_PER_HEAD}


def _kv_rows(x: torch.Tensor, heads: int, head_dim: int, name: str):
    """(n, ld) of a [n, heads*head_dim] or [n, heads, head_dim] device tensor
    whose heads are packed back to back within a token."""
    if not x.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if x.dim() == 3:
        if tuple(x.shape[1:]) != (heads, head_dim) or x.stride(2) != 1 or (heads > 1 and x.stride(1) != head_dim):
            raise ValueError("%s [n, heads, head_dim] must have packed heads" % name)
    elif x.dim() == 2:
        if x.shape[1] != heads * head_dim or (x.shape[1] > 1 and x.stride(1) != 1):
            raise ValueError("%s must be [n, %d] with a contiguous last dimension" % (name, heads * head_dim))
    else:
        raise ValueError("%s must be 2-D or 3-D" % name)
    n = x.shape[0]
    return n, (x.stride(0) if n > 1 else heads * head_dim)


def _kv_scales(scale_inv: Optional[torch.Tensor], storage: str, scaling: str, capacity: int, heads: int,
               device: torch.device):
    """Pointer of a cache's scales: [capacity, heads] per (token, head), [heads]
    fixed per head; none for bf16 storage (the library reports a missing one)."""
    if scale_inv is None or storage == "bf16":
        return _ptr(scale_inv)
    n = capacity * heads if scaling == "token_head" else heads
    return _buf(scale_inv, n, torch.float32, device, "scale_inv")


def _slots(slots: Optional[torch.Tensor], n: int):
    if slots is None:
        return None
    if slots.dtype != torch.int64 or not slots.is_cuda or slots.shape != (n,) or not slots.is_contiguous():
        raise ValueError("slots must be a contiguous int64 device tensor of %d entries" % n)
    return slots.data_ptr()


def kv_store(x: torch.Tensor, cache: torch.Tensor, scale_inv: Optional[torch.Tensor], storage="e4m3",
             scaling="token_head", slots: Optional[torch.Tensor] = None, pow2: bool = False,
             diag: Optional[Diag] = None) -> None:
    """Store new tokens' vectors x [n, heads*head_dim] (bf16/fp32) into one
    layer's cache [capacity, heads, head_dim] (uint8 codes, bf16 for the
    "bf16" storage) at rows `slots` (None: rows 0..n-1; negative = padding)."""
    capacity, heads, head_dim = cache.shape
    n, ld = _kv_rows(x, heads, head_dim, "x")
    if x.dtype == torch.bfloat16:
        in_dt = _lib.FP8_IN_BF16
    elif x.dtype == torch.float32:
        in_dt = _lib.FP8_IN_F32
    else:
        raise TypeError("x must be bfloat16 or float32, got %s" % x.dtype)
    want = torch.bfloat16 if storage == "bf16" else torch.uint8
    if cache.dtype != want or not cache.is_contiguous():
        raise ValueError("cache must be a contiguous %s tensor" % want)
    _same_device(x, cache.device, "x")
    if slots is not None:
        _same_device(slots, cache.device, "slots")
    st = _lib.lib().fp8_kv_store(
        x.data_ptr(), in_dt, n, ld, heads, head_dim, _slots(slots, n), KV_STORAGE[storage],
        KV_SCALING[scaling], _lib.FP8_SCALE_POW2 if pow2 else 0, cache.data_ptr(),
        _kv_scales(scale_inv, storage, scaling, capacity, heads, cache.device), capacity,
        _ptr(diag.buf) if diag is not None else None, _stream(cache.device))
    _lib.check(st, "fp8_kv_store")


def kv_load(cache: torch.Tensor, scale_inv: Optional[torch.Tensor], n: Optional[int] = None, storage="e4m3",
            scaling="token_head", slots: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gather n cache rows (slots, or rows 0..n-1) as dequantized values
    out [n, heads*head_dim] (bf16 or fp32)."""
    capacity, heads, head_dim = cache.shape
    if n is None:
        n = slots.shape[0] if slots is not None else capacity
    if out is None:
        out = torch.empty((n, heads * head_dim), dtype=out_dtype, device=cache.device)
    n2, ld_out = _kv_rows(out, heads, head_dim, "out")
    if n2 != n:
        raise ValueError("out has %d rows, expected %d" % (n2, n))
    _same_device(out, cache.device, "out")
    if slots is not None:
        _same_device(slots, cache.device, "slots")
    st = _lib.lib().fp8_kv_load(
        cache.data_ptr(), KV_STORAGE[storage], KV_SCALING[scaling],
        _kv_scales(scale_inv, storage, scaling, capacity, heads, cache.device), capacity, heads, head_dim,
        _slots(slots, n), n, _out_dtype(out.dtype), out.data_ptr(), ld_out, _stream(cache.device))
    _lib.check(st, "fp8_kv_load")
    return out


class KVTensorCache:
    """One layer's K (or V) cache: `data` [capacity, heads, head_dim] (uint8
    codes; bf16 for the "bf16" storage) and `scale_inv` ([capacity, heads] for
    per-(token, head) scales, [heads] fixed scales for "head" scaling)."""

    def __init__(self, capacity: int, heads: int, head_dim: int, storage="e4m3", scaling="token_head",
                 head_scale_inv: Optional[torch.Tensor] = None, device="cuda"):
        if storage not in KV_STORAGE or scaling not in KV_SCALING:
            raise ValueError("storage %r / scaling %r" % (storage, scaling))
        self.storage, self.scaling = storage, scaling
        self.capacity, self.heads, self.head_dim = capacity, heads, head_dim
        dt = torch.bfloat16 if storage == "bf16" else torch.uint8
        self.data = torch.zeros((capacity, heads, head_dim), dtype=dt, device=device)
        if storage == "bf16":
            self.scale_inv = None
        elif scaling == "token_head":
            self.scale_inv = torch.zeros((capacity, heads), dtype=torch.float32, device=device)
        else:
            if head_scale_inv is None or head_scale_inv.numel() != heads:
                raise ValueError("'head' scaling needs head_scale_inv with %d entries" % heads)
            self.scale_inv = head_scale_inv.to(device=device, dtype=torch.float32).contiguous()

    @property
    def nbytes(self) -> int:
        n = self.data.numel() * self.data.element_size()
        return n + (self.scale_inv.numel() * 4 if self.scale_inv is not None else 0)

    def store(self, x: torch.Tensor, slots: Optional[torch.Tensor] = None, pow2: bool = False,
              diag: Optional[Diag] = None) -> None:
        kv_store(x, self.data, self.scale_inv, self.storage, self.scaling, slots, pow2, diag)

    def load(self, n: Optional[int] = None, slots: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
        return kv_load(self.data, self.scale_inv, n, self.storage, self.scaling, slots, out_dtype, out)


class KVCache:
    """K and V caches of every layer of a model.  Layers listed in
    `bf16_k_layers` keep their K cache in bf16 (the per-layer fallback of a
    precision-sensitive layer); `bf16_v_layers` likewise for V."""

    def __init__(self, layers: int, capacity: int, kv_heads: int, head_dim: int, storage="e4m3",
                 scaling="token_head", bf16_k_layers=(), bf16_v_layers=(), head_scale_inv=None, device="cuda"):
        bk, bv = set(bf16_k_layers), set(bf16_v_layers)
        for s in (bk, bv):
            if any(not 0 <= i < layers for i in s):
                raise ValueError("fallback layer index out of range 0..%d" % (layers - 1))

        def make(i, fallback, which):
            st = "bf16" if i in fallback else storage
            hs = None if head_scale_inv is None else head_scale_inv[which][i]
            return KVTensorCache(capacity, kv_heads, head_dim, st, scaling, hs, device)

        self.k = [make(i, bk, 0) for i in range(layers)]
        self.v = [make(i, bv, 1) for i in range(layers)]

    @property
    def nbytes(self) -> int:
        return sum(c.nbytes for c in self.k + self.v)

    def store(self, layer: int, k: torch.Tensor, v: torch.Tensor, slots: Optional[torch.Tensor] = None,
              pow2: bool = False) -> None:
        self.k[layer].store(k, slots, pow2)
        self.v[layer].store(v, slots, pow2)

    def load(self, layer: int, n: Optional[int] = None, slots: Optional[torch.Tensor] = None,
             out_dtype=torch.bfloat16):
        return (self.k[layer].load(n, slots, out_dtype), self.v[layer].load(n, slots, out_dtype))
