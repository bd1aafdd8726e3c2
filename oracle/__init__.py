"""CPU oracle for FP8 scaled quantization and the scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  It shares
no code with the HIP library (``fp8_precision_quantization_amd``) and never
imports it; the library never imports this.

The arithmetic lives in ``fp8_oracle.c`` (plain C, IEEE binary32/binary64,
no FMA contraction).  This module only marshals numpy arrays.  Every function
cites the passage of the web pages it follows in the C source.

Functions with no pin against something other than themselves: none.  Every
function here is pinned by ``tests/test_oracle_pins.py``,
``tests/test_oracle_kv_pins.py`` or ``tests/test_oracle_grouped_pins.py``
(library routines, closed forms, page constants, exact integer arithmetic,
brute force).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

E4M3, E5M2 = 0, 1
GRAN_TENSOR, GRAN_ROW, GRAN_1x128, GRAN_128x128 = 0, 1, 2, 3
IN_F32, IN_BF16 = 0, 1
KV_E4M3, KV_E5M2, KV_BF16 = 0, 1, 2
KV_PER_TOKEN_HEAD, KV_PER_HEAD = 0, 1

GCC_FLAGS = ["-O2", "-std=gnu11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
             "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        f32 = ctypes.c_float
        L.or_decode.restype = ctypes.c_double
        L.or_decode.argtypes = [i32, ctypes.c_uint8]
        L.or_decode_table.argtypes = [i32, P]
        L.or_format_max.restype = ctypes.c_double
        L.or_format_max.argtypes = [i32]
        L.or_encode.restype = ctypes.c_uint8
        L.or_encode.argtypes = [i32, f32]
        L.or_encode_array.argtypes = [i32, P, i64, P]
        L.or_num_groups.restype = i64
        L.or_num_groups.argtypes = [i32, i64, i64]
        L.or_amax.argtypes = [P, i32, i64, i64, i64, i32, P]
        L.or_scale.argtypes = [f32, i32, i32, P, P]
        L.or_quantize_with_scales.argtypes = [P, i32, i64, i64, i64, i32, i32, P, P, i64, P]
        L.or_quantize.argtypes = [P, i32, i64, i64, i64, i32, i32, i32, P, i64, P, P, P, P]
        L.or_ring_init.argtypes = [P, ctypes.c_int32]
        L.or_ring_window_max.restype = f32
        L.or_ring_window_max.argtypes = [P]
        L.or_delayed_step.argtypes = [P, P, i32, i64, i64, i64, i32, P, i64, f32, P, P]
        L.or_gemm_sampled.argtypes = [P, i32, i64, P, i32, i64, i64, P, i32, P, i32, P, P, i64, P, P]
        L.or_gemm.argtypes = [P, i32, i64, P, i32, i64, i64, i64, i64, P, i32, P, i32, P, i64, P, i64]
        L.or_blockgemm_sampled.argtypes = [P, i64, P, i64, i64, P, P, P, P, i64, P, P]
        L.or_blockgemm.argtypes = [P, i64, P, i64, i64, i64, i64, P, P, P, i64, P, i64]
        L.or_gemm_exact_sampled.argtypes = [P, i32, i64, P, i32, i64, i64, P, i32, P, i32, i32,
                                            P, P, i64, P]
        L.or_f32_to_bf16.restype = ctypes.c_uint16
        L.or_f32_to_bf16.argtypes = [f32]
        L.or_f32_to_bf16_array.argtypes = [P, i64, P]
        L.or_kv_store.argtypes = [P, i32, i64, i64, i64, i64, P, i64, i32, i32, i32, P, P, P]
        L.or_kv_load.argtypes = [P, i32, i32, P, i64, i64, i64, P, i64, i32, P, i64]
        L.or_num_threads.restype = i32
        L.or_num_threads.argtypes = []
        L.or_set_num_threads.restype = None
        L.or_set_num_threads.argtypes = [i32]
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().or_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (for timing it; results do not
    depend on the thread count)."""
    lib().or_set_num_threads(int(n))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _in_array(x: np.ndarray):
    """Return (contiguous array, dtype code).  bf16 data travels as uint16."""
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), IN_F32
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), IN_BF16
    raise TypeError("oracle inputs are float32 or bf16 bit patterns (uint16)")


def fmt_code(fmt) -> int:
    if fmt in (E4M3, "e4m3"):
        return E4M3
    if fmt in (E5M2, "e5m2"):
        return E5M2
    raise ValueError(fmt)


GRAN_NAMES = {"tensor": GRAN_TENSOR, "row": GRAN_ROW, "1x128": GRAN_1x128,
              "128x128": GRAN_128x128}


def gran_code(g) -> int:
    return GRAN_NAMES[g] if isinstance(g, str) else int(g)


# ----------------------------------------------------------------- codec --
def decode_table(fmt) -> np.ndarray:
    out = np.empty(256, dtype=np.float64)
    lib().or_decode_table(fmt_code(fmt), _p(out))
    return out


def format_max(fmt) -> float:
    return lib().or_format_max(fmt_code(fmt))


def encode(fmt, v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().or_encode_array(fmt_code(fmt), _p(v), v.size, _p(out))
    return out


# ---------------------------------------------------------- amax / scale --
def group_grid(gran, rows: int, cols: int):
    g = gran_code(gran)
    if g == GRAN_TENSOR:
        return (1, 1)
    if g == GRAN_ROW:
        return (rows, 1)
    if g == GRAN_1x128:
        return (rows, (cols + 127) // 128)
    return ((rows + 127) // 128, (cols + 127) // 128)


def amax(x: np.ndarray, gran="tensor") -> np.ndarray:
    x, dt = _in_array(x)
    rows, cols = x.shape
    out = np.empty(group_grid(gran, rows, cols), dtype=np.float32)
    lib().or_amax(_p(x), dt, rows, cols, cols, gran_code(gran), _p(out))
    return out


def scale(amax_value: float, fmt, pow2: bool = False):
    s = np.empty(1, dtype=np.float32)
    si = np.empty(1, dtype=np.float32)
    lib().or_scale(float(amax_value), fmt_code(fmt), int(bool(pow2)), _p(s), _p(si))
    return s[0], si[0]


def quantize(x: np.ndarray, fmt, gran="tensor", pow2: bool = False):
    """Just-in-time quantize.  Returns dict with q, amax, scale, scale_inv and
    counts (sat, nonfinite, underflow)."""
    x, dt = _in_array(x)
    rows, cols = x.shape
    grid = group_grid(gran, rows, cols)
    q = np.empty((rows, cols), dtype=np.uint8)
    am = np.empty(grid, dtype=np.float32)
    s = np.empty(grid, dtype=np.float32)
    si = np.empty(grid, dtype=np.float32)
    counts = np.zeros(3, dtype=np.int64)
    lib().or_quantize(_p(x), dt, rows, cols, cols, gran_code(gran), fmt_code(fmt),
                      int(bool(pow2)), _p(q), cols, _p(am), _p(s), _p(si), _p(counts))
    return {"q": q, "amax": am, "scale": s, "scale_inv": si,
            "sat": int(counts[0]), "nonfinite": int(counts[1]), "underflow": int(counts[2])}


def quantize_with_scales(x: np.ndarray, fmt, gran, scales: np.ndarray):
    x, dt = _in_array(x)
    rows, cols = x.shape
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    q = np.empty((rows, cols), dtype=np.uint8)
    counts = np.zeros(3, dtype=np.int64)
    lib().or_quantize_with_scales(_p(x), dt, rows, cols, cols, gran_code(gran), fmt_code(fmt),
                                  _p(scales), _p(q), cols, _p(counts))
    return q, {"sat": int(counts[0]), "nonfinite": int(counts[1]), "underflow": int(counts[2])}


# ------------------------------------------------------------ delayed ring --
class _Ring(ctypes.Structure):
    _fields_ = [("amax", ctypes.c_float * 16), ("len", ctypes.c_int32),
                ("pos", ctypes.c_int32), ("count", ctypes.c_int32)]


class DelayedScaler:
    """Amax-history ring for one tensor (see or_delayed_step in the C source).
    spike_threshold > 0 enables the spike guard of or_delayed_step."""

    def __init__(self, fmt, length: int = 16, spike_threshold: float = 0.0):
        assert 1 <= length <= 16
        self.fmt = fmt_code(fmt)
        self.spike_threshold = float(spike_threshold)
        self.ring = _Ring()
        lib().or_ring_init(ctypes.byref(self.ring), length)

    def window_max(self) -> float:
        return lib().or_ring_window_max(ctypes.byref(self.ring))

    def step(self, x: np.ndarray):
        x, dt = _in_array(x)
        rows, cols = x.shape
        q = np.empty((rows, cols), dtype=np.uint8)
        out4 = np.zeros(4, dtype=np.float32)
        counts = np.zeros(3, dtype=np.int64)
        lib().or_delayed_step(ctypes.byref(self.ring), _p(x), dt, rows, cols, cols, self.fmt,
                              _p(q), cols, ctypes.c_float(self.spike_threshold), _p(out4), _p(counts))
        return {"q": q, "scale": out4[0], "scale_inv": out4[1], "amax": out4[2],
                "spiked": bool(out4[3]), "sat": int(counts[0]), "nonfinite": int(counts[1]),
                "underflow": int(counts[2])}

    def state(self):
        return {"amax": np.array(self.ring.amax[:], dtype=np.float32),
                "len": self.ring.len, "pos": self.ring.pos, "count": self.ring.count}


# ------------------------------------------------------------------ GEMM --
def _scale_arg(s, n):
    """A scalar scale (size 1) or one scale per row (size n)."""
    s = np.ascontiguousarray(np.atleast_1d(np.asarray(s, dtype=np.float32)).ravel())
    if s.size == 1:
        return s, 0
    if s.size != n:
        raise ValueError("scale vector has %d entries, expected 1 or %d" % (s.size, n))
    return s, 1


def gemm(A: np.ndarray, fa, B: np.ndarray, fb, a_inv, b_inv, with_p: bool = True):
    """Full dequantized fp32 GEMM Y = A_hat . B_hat^T (A: [M,K], B: [N,K])."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    sa, apr = _scale_arg(a_inv, M)
    sb, bpr = _scale_arg(b_inv, N)
    Y = np.empty((M, N), dtype=np.float32)
    P = np.empty((M, N), dtype=np.float64) if with_p else None
    lib().or_gemm(_p(A), fmt_code(fa), K, _p(B), fmt_code(fb), K, M, N, K, _p(sa), apr,
                  _p(sb), bpr, _p(Y), N, _p(P) if with_p else None, N)
    return (Y, P) if with_p else Y


def gemm_sampled(A, fa, B, fb, a_inv, b_inv, ms, ns):
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    M, K = A.shape
    N, _ = B.shape
    sa, apr = _scale_arg(a_inv, M)
    sb, bpr = _scale_arg(b_inv, N)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    y = np.empty(ms.size, dtype=np.float32)
    p = np.empty(ms.size, dtype=np.float64)
    lib().or_gemm_sampled(_p(A), fmt_code(fa), K, _p(B), fmt_code(fb), K, K, _p(sa), apr,
                          _p(sb), bpr, _p(ms), _p(ns), ms.size, _p(y), _p(p))
    return y, p


def blockgemm_sampled(A, B, a_inv, b_inv, ms, ns):
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    M, K = A.shape
    assert K % 128 == 0
    a_inv = np.ascontiguousarray(a_inv, dtype=np.float32)
    b_inv = np.ascontiguousarray(b_inv, dtype=np.float32)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    y = np.empty(ms.size, dtype=np.float32)
    p = np.empty(ms.size, dtype=np.float64)
    lib().or_blockgemm_sampled(_p(A), K, _p(B), K, K, _p(a_inv), _p(b_inv), _p(ms), _p(ns),
                               ms.size, _p(y), _p(p))
    return y, p


def blockgemm(A, B, a_inv, b_inv, with_p: bool = True):
    """Full block-scaled GEMM (A: [M,K] with a_inv [M, K/128]; B: [N,K] with
    b_inv [N/128, K/128]; K % 128 == 0)."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2 and K % 128 == 0
    a_inv = np.ascontiguousarray(a_inv, dtype=np.float32)
    b_inv = np.ascontiguousarray(b_inv, dtype=np.float32)
    assert a_inv.size == M * (K // 128) and b_inv.size == ((N + 127) // 128) * (K // 128)
    Y = np.empty((M, N), dtype=np.float32)
    P = np.empty((M, N), dtype=np.float64) if with_p else None
    lib().or_blockgemm(_p(A), K, _p(B), K, M, N, K, _p(a_inv), _p(b_inv), _p(Y), N,
                       _p(P) if with_p else None, N)
    return (Y, P) if with_p else Y


def gemm_exact_sampled(A, fa, B, fb, a_inv, b_inv, ms, ns, block_mode=False):
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    M, K = A.shape
    N, _ = B.shape
    if block_mode:
        sa = np.ascontiguousarray(a_inv, dtype=np.float32)
        sb = np.ascontiguousarray(b_inv, dtype=np.float32)
        apr = bpr = 1
    else:
        sa, apr = _scale_arg(a_inv, M)
        sb, bpr = _scale_arg(b_inv, N)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    y = np.empty(ms.size, dtype=np.float64)
    lib().or_gemm_exact_sampled(_p(A), fmt_code(fa), K, _p(B), fmt_code(fb), K, K, _p(sa), apr,
                                _p(sb), bpr, int(block_mode), _p(ms), _p(ns), ms.size, _p(y))
    return y


# ------------------------------------------------------------- bf16 out --
def f32_to_bf16(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().or_f32_to_bf16_array(_p(v), v.size, _p(out))
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# -------------------------------------------------------------- KV cache --
_KV_STORAGE = {"e4m3": KV_E4M3, "e5m2": KV_E5M2, "bf16": KV_BF16}
_KV_SCALING = {"token_head": KV_PER_TOKEN_HEAD, "head": KV_PER_HEAD}


def _slots_arg(slots, n):
    if slots is None:
        return None
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    assert slots.shape == (n,)
    return slots


def kv_store(x: np.ndarray, heads: int, head_dim: int, cache: np.ndarray, scale_inv: np.ndarray,
             storage="e4m3", scaling="token_head", slots=None, pow2: bool = False):
    """Store n new tokens (x: [n x heads*head_dim], float32 or bf16 bits) into
    a cache in place (see or_kv_store).  cache: uint8 [capacity x heads x
    head_dim] (uint16 for bf16 storage); scale_inv: float32 [capacity x heads]
    (written, token_head) or [heads] (read, head).  Returns the counters."""
    x, dt = _in_array(x)
    n = x.shape[0]
    assert x.shape[1] == heads * head_dim
    st = _KV_STORAGE[storage]
    sc = _KV_SCALING[scaling]
    capacity = cache.shape[0]
    assert cache.flags.c_contiguous and cache.shape[1:] == (heads, head_dim)
    assert cache.dtype == (np.uint16 if st == KV_BF16 else np.uint8)
    assert scale_inv.dtype == np.float32 and scale_inv.flags.c_contiguous
    sl = _slots_arg(slots, n)
    counts = np.zeros(3, dtype=np.int64)
    lib().or_kv_store(_p(x), dt, n, heads, head_dim, x.shape[1], _p(sl) if sl is not None else None,
                      capacity, st, sc, int(bool(pow2)), _p(cache), _p(scale_inv), _p(counts))
    return {"sat": int(counts[0]), "nonfinite": int(counts[1]), "underflow": int(counts[2])}


def kv_load(cache: np.ndarray, scale_inv: np.ndarray, n: int, storage="e4m3",
            scaling="token_head", slots=None, out_bf16: bool = True, out=None):
    """Gather n cache rows and dequantize them (see or_kv_load).  Returns
    out: [n x heads*head_dim], uint16 bf16 bits or float32."""
    st = _KV_STORAGE[storage]
    sc = _KV_SCALING[scaling]
    capacity, heads, head_dim = cache.shape
    assert cache.flags.c_contiguous
    scale_inv = np.ascontiguousarray(scale_inv, dtype=np.float32)
    if out is None:
        out = np.zeros((n, heads * head_dim), dtype=np.uint16 if out_bf16 else np.float32)
    assert out.flags.c_contiguous and out.shape == (n, heads * head_dim)
    sl = _slots_arg(slots, n)
    lib().or_kv_load(_p(cache), st, sc, _p(scale_inv), n, heads, head_dim,
                     _p(sl) if sl is not None else None, capacity, int(bool(out_bf16)),
                     _p(out), heads * head_dim)
    return out


# ----------------------------------------------------------- grouped GEMM --
def group_of_rows(offsets, ms) -> np.ndarray:
    """Route rows to groups ("DeepL bets on FP8" (hmyw.cn) 3.2: the tokens of
    a batch split into groups by their routing, each group multiplied with
    its own expert's weight).  READING: group g holds rows [offsets[g],
    offsets[g+1]) of the token matrix (offsets non-decreasing); a row outside
    every group gets -1 (no output)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    ms = np.asarray(ms, dtype=np.int64)
    g = np.searchsorted(offsets, ms, side="right") - 1
    G = offsets.size - 1
    inside = (g >= 0) & (g < G)
    inside &= ms < offsets[np.clip(g + 1, 0, G)]
    return np.where(inside, g, -1)


def grouped_gemm_sampled(A, fa, B, fb, offsets, a_inv, b_inv, ms, ns, exact=False):
    """Grouped scaled GEMM at sampled outputs: C[m, n] = the scaled GEMM of
    row m of A with expert g(m)'s weight B[g] ([G, N, K]), its scale b_inv[g]
    (one per expert, [G]) or b_inv[g, n] ([G, N]); a_inv is one scale or one
    per row of A.  Each group is the plain sampled GEMM (gemm_sampled, or
    gemm_exact_sampled with exact=True) on its own rows.  Rows outside every
    group give NaN."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    G, N, K = B.shape
    b_inv = np.asarray(b_inv, dtype=np.float32).reshape(G, -1)
    assert b_inv.shape[1] in (1, N)
    ms = np.asarray(ms, dtype=np.int64)
    ns = np.asarray(ns, dtype=np.int64)
    g = group_of_rows(offsets, ms)
    y = np.full(ms.size, np.nan, dtype=np.float64 if exact else np.float32)
    p = np.full(ms.size, np.nan, dtype=np.float64)
    for gi in np.unique(g[g >= 0]):
        sel = np.nonzero(g == gi)[0]
        if exact:
            y[sel] = gemm_exact_sampled(A, fa, B[gi], fb, a_inv, b_inv[gi], ms[sel], ns[sel])
        else:
            y[sel], p[sel] = gemm_sampled(A, fa, B[gi], fb, a_inv, b_inv[gi], ms[sel], ns[sel])
    return y if exact else (y, p)
