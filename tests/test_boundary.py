"""Boundary checks that run without a GPU: the C-ABI library loads, exports
every function include/fp8mi.h declares, and rejects invalid arguments
before any device call (validation precedes the device check, so these
calls never touch HIP).  Pointer values here are fake and never
dereferenced: every call fails validation first."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import pytest

from fp8_precision_quantization_amd import _lib

L = _lib


def test_library_exports_every_header_function():
    lib = L.lib()
    declared = L.header_functions()
    assert set(declared) == set(L.SIGNATURES), declared
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared) <= exported


def test_library_never_allocates_or_synchronizes():
    """The caller owns every buffer: the library imports no HIP allocation,
    free, memset or synchronization routine."""
    out = subprocess.run(["nm", "-D", "--undefined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    imported = {ln.split()[-1].split("@")[0] for ln in out.splitlines() if ln.strip()}
    assert any(s.startswith("hipLaunchKernel") for s in imported), sorted(imported)
    forbidden = [s for s in imported
                 if s.startswith(("hipMalloc", "hipFree", "hipExtMalloc", "hipHostMalloc", "hipMemset",
                                  "hipDeviceSynchronize", "hipStreamSynchronize", "hipEventSynchronize",
                                  "hipMemcpy", "hipMallocAsync", "hipMemPool"))]
    assert forbidden == [], forbidden


def test_library_is_gfx950_only_code_object():
    out = subprocess.run(["strings", "-n", "8", L.LIB_PATH], capture_output=True, text=True).stdout
    assert "gfx950" in out
    for other in ("gfx942", "gfx90a", "gfx1100", "sm_"):
        assert "amdgcn-amd-amdhsa--" + other not in out


def test_abi_version_and_status_strings():
    lib = L.lib()
    assert lib.fp8_abi_version() == 7
    assert lib.fp8_workspace_size() == L.WORKSPACE_BYTES
    for code, name in [(0, "FP8_OK"), (1, "FP8_ERR_INVALID_ARG"), (2, "FP8_ERR_UNSUPPORTED_SHAPE"),
                       (3, "FP8_ERR_MISALIGNED"), (4, "FP8_ERR_UNSUPPORTED_DEVICE"), (5, "FP8_ERR_HIP")]:
        assert L.status_name(code) == name


FAKE = 0x10000          # 64 KiB-aligned fake device address, never dereferenced


def q(**kw):
    a = dict(x=FAKE, in_dt=L.FP8_IN_BF16, rows=64, cols=64, ld=64, fmt=L.FP8_E4M3,
             gran=L.FP8_GRAN_TENSOR, flags=0, hist=None, q=FAKE, ldq=64, sinv=FAKE, amax=FAKE,
             diag=None, ws=FAKE, ws_bytes=L.WORKSPACE_BYTES)
    a.update(kw)
    st = L.lib().fp8_quantize(a["x"], a["in_dt"], a["rows"], a["cols"], a["ld"], a["fmt"], a["gran"],
                              a["flags"], a["hist"], a["q"], a["ldq"], a["sinv"], a["amax"], a["diag"],
                              a["ws"], a["ws_bytes"], None)
    return st, L.lib().fp8_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x=None), 1, "x is NULL"),
    (dict(in_dt=7), 1, "in_dtype"),
    (dict(rows=-1), 1, "negative"),
    (dict(ld=32), 1, "ld="),
    (dict(fmt=3), 1, "format"),
    (dict(gran=9), 1, "granularity"),
    (dict(flags=8), 1, "flag"),
    (dict(flags=2, gran=1), 1, "TRANSPOSE"),
    (dict(hist=FAKE, gran=2), 1, "delayed"),
    (dict(q=None), 1, "q is NULL"),
    (dict(ldq=10), 1, "ldq"),
    (dict(flags=2, rows=100, ldq=64), 1, "ldq"),
    (dict(sinv=None), 1, "scale_inv_out"),
    (dict(amax=None), 1, "amax_out"),
    (dict(x=FAKE + 1), 3, "aligned"),
    (dict(in_dt=L.FP8_IN_F32, x=FAKE + 2), 3, "aligned"),
    (dict(hist=FAKE + 4), 3, "hist"),
    (dict(amax=FAKE + 2), 3, "aligned"),
    (dict(rows=2 ** 32), 2, "2^31"),
    (dict(flags=4), 1, "FP8_SPIKE_GUARD"),
    (dict(flags=16), 1, "flag"),
    (dict(ws=None), 1, "workspace is NULL"),
    (dict(ws_bytes=L.WORKSPACE_BYTES - 16), 1, "workspace_bytes"),
    (dict(ws=FAKE + 8), 3, "workspace"),
])
def test_quantize_validation(kw, status, needle):
    st, msg = q(**kw)
    assert st == status, (st, msg)
    assert needle in msg


def qd(**kw):
    a = dict(x=FAKE, in_dt=L.FP8_IN_BF16, rows=64, cols=96, ld=96, fmt=L.FP8_E5M2, flags=0, hist=None,
             q=FAKE, ldq=96, qt=FAKE, ldqt=64, sinv=FAKE, amax=FAKE, diag=None, ws=FAKE,
             ws_bytes=L.WORKSPACE_BYTES)
    a.update(kw)
    st = L.lib().fp8_quantize_dual(a["x"], a["in_dt"], a["rows"], a["cols"], a["ld"], a["fmt"], a["flags"],
                                   a["hist"], a["q"], a["ldq"], a["qt"], a["ldqt"], a["sinv"], a["amax"],
                                   a["diag"], a["ws"], a["ws_bytes"], None)
    return st, L.lib().fp8_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), 1, "q is NULL"),
    (dict(qt=None), 1, "qt is NULL"),
    (dict(ldq=90), 1, "ldq"),
    (dict(ldqt=60), 1, "ldqt"),
    (dict(flags=2), 1, "flag"),
    (dict(flags=4), 1, "FP8_SPIKE_GUARD"),
    (dict(fmt=5), 1, "format"),
    (dict(x=FAKE + 1), 3, "aligned"),
    (dict(ws=None), 1, "workspace is NULL"),
])
def test_quantize_dual_validation(kw, status, needle):
    st, msg = qd(**kw)
    assert st == status, (st, msg)
    assert needle in msg


def qt(descs=None, count=None, in_dt=L.FP8_IN_BF16, fmt=L.FP8_E4M3, flags=0, ws=FAKE,
       ws_bytes=L.WORKSPACE_BYTES, **kw):
    """fp8_quantize_tensors on two fake 64 x 96 tensors; kw overrides fields
    of tensor 1 (the second), so errors must name index 1."""
    if descs is None:
        descs = [dict(x=FAKE, rows=64, cols=96, q=FAKE, scale_inv=FAKE, amax=FAKE, diag=None) for _ in range(2)]
        descs[1].update(kw)
    arr = (L.Fp8Tensor * max(len(descs), 1))(*[L.Fp8Tensor(**d) for d in descs])
    ptr = ctypes.cast(arr, ctypes.c_void_p) if descs else None
    st = L.lib().fp8_quantize_tensors(ptr, len(descs) if count is None else count, in_dt, fmt, flags, ws,
                                      ws_bytes, None)
    return st, L.lib().fp8_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x=None), 1, "tensor 1: x is NULL"),
    (dict(q=None), 1, "tensor 1: q is NULL"),
    (dict(scale_inv=None), 1, "tensor 1: scale_inv is NULL"),
    (dict(amax=None), 1, "tensor 1: amax is NULL"),
    (dict(rows=-2), 1, "tensor 1: negative"),
    (dict(cols=2 ** 31 + 1), 2, "tensor 1: rows and cols"),
    (dict(rows=2 ** 31, cols=2 ** 31), 2, "tensor 1 too large"),
    (dict(x=FAKE + 8), 3, "tensor 1: x must be 16-byte aligned"),
    (dict(q=FAKE + 4), 3, "tensor 1: q must be 8-byte aligned"),
    (dict(amax=FAKE + 2), 3, "tensor 1: scale_inv and amax"),
    (dict(diag=FAKE + 2), 3, "tensor 1: diag"),
    (dict(in_dt=9), 1, "in_dtype"),
    (dict(fmt=4), 1, "format"),
    (dict(flags=2), 1, "FP8_SCALE_POW2"),
    (dict(flags=4), 1, "FP8_SCALE_POW2"),
    (dict(ws=None), 1, "workspace is NULL"),
    (dict(ws_bytes=1024), 1, "workspace_bytes"),
    (dict(ws=FAKE + 4), 3, "workspace"),
    (dict(count=0), 1, "count=0"),
    (dict(count=9), 1, "count=9"),
])
def test_quantize_tensors_validation(kw, status, needle):
    top = {k: kw.pop(k) for k in ("in_dt", "fmt", "flags", "ws", "ws_bytes", "count") if k in kw}
    st, msg = qt(**top, **kw)
    assert st == status, (st, msg)
    assert needle in msg


def test_quantize_tensors_null_array_and_empty_tensors_validate():
    st, msg = qt(descs=[], count=1)
    assert st == 1 and "tensors is NULL" in msg
    # empty tensors need no x or q; validation then reaches the device check
    # (no GPU here), never a launch
    st, msg = qt(x=None, q=None, rows=0)
    assert st in (L.FP8_ERR_UNSUPPORTED_DEVICE, L.FP8_ERR_HIP), (st, msg)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_tensor_descriptor_layout_matches_header(tmp_path):
    """The binding's fp8_tensor (ctypes) has the header's size and offsets."""
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "fp8mi.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu %zu %zu %zu %zu %d\\n", sizeof(fp8_tensor), '
                   'offsetof(fp8_tensor, x), offsetof(fp8_tensor, rows), offsetof(fp8_tensor, cols), '
                   'offsetof(fp8_tensor, q), offsetof(fp8_tensor, scale_inv), offsetof(fp8_tensor, amax), '
                   'offsetof(fp8_tensor, diag), FP8_MAX_TENSORS); return 0; }\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(L.HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    T = L.Fp8Tensor
    want = [ctypes.sizeof(T)] + [getattr(T, f).offset for f, _ in T._fields_] + [L.MAX_TENSORS]
    assert got == want


def gg(**kw):
    a = dict(A=FAKE, fa=0, lda=256, B=FAKE, fb=0, ldb=256, gstride=512 * 256, M=1000, N=512, K=256, G=8,
             offs=FAKE, sa=FAKE, sa_row=1, sb=FAKE, sb_row=0, C=FAKE, out_dt=L.FP8_OUT_BF16, ldc=512,
             ws=FAKE, ws_bytes=L.WORKSPACE_BYTES)
    a.update(kw)
    st = L.lib().fp8_grouped_gemm(a["A"], a["fa"], a["lda"], a["B"], a["fb"], a["ldb"], a["gstride"], a["M"], a["N"],
                                  a["K"], a["G"], a["offs"], a["sa"], a["sa_row"], a["sb"], a["sb_row"], a["C"],
                                  a["out_dt"], a["ldc"], a["ws"], a["ws_bytes"], None)
    return st, L.lib().fp8_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(fa=2), 1, "formats"),
    (dict(sb_row=2), 1, "per_row"),
    (dict(K=100, lda=112, ldb=112, gstride=512 * 112), 2, "multiple of 16"),
    (dict(G=0), 1, "groups="),
    (dict(offs=None), 1, "group_offsets is NULL"),
    (dict(offs=FAKE + 2), 3, "group_offsets"),
    (dict(gstride=511 * 256), 1, "b_group_stride"),
    (dict(gstride=511 * 256 + 256 + 8), 3, "b_group_stride"),
    (dict(M=256 * 1980, G=4), 2, "FP8_GROUPED_MAX_TILES"),
    (dict(G=1984, M=0), 2, "FP8_GROUPED_MAX_TILES"),
    (dict(C=None), 1, "C is NULL"),
    (dict(lda=128), 1, "lda"),
    (dict(ws=None), 1, "workspace is NULL"),
    (dict(ws_bytes=100), 1, "workspace_bytes"),
])
def test_grouped_gemm_validation(kw, status, needle):
    st, msg = gg(**kw)
    assert st == status, (st, msg)
    assert needle in msg


def kvs(**kw):
    a = dict(x=FAKE, in_dt=L.FP8_IN_BF16, n=16, ld=1024, heads=8, hd=128, slots=None, storage=L.FP8_KV_E4M3,
             scaling=L.FP8_KV_PER_TOKEN_HEAD, flags=0, cache=FAKE, sinv=FAKE, cap=64, diag=None)
    a.update(kw)
    st = L.lib().fp8_kv_store(a["x"], a["in_dt"], a["n"], a["ld"], a["heads"], a["hd"], a["slots"], a["storage"],
                              a["scaling"], a["flags"], a["cache"], a["sinv"], a["cap"], a["diag"], None)
    return st, L.lib().fp8_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(storage=3), 1, "storage"),
    (dict(scaling=2), 1, "scaling"),
    (dict(n=-1), 1, "negative"),
    (dict(cap=-1), 1, "negative"),
    (dict(hd=100), 2, "head_dim"),
    (dict(hd=2056, ld=8 * 2056), 2, "head_dim"),
    (dict(hd=0), 2, "head_dim"),
    (dict(n=2 ** 28), 2, "2^31"),
    (dict(cache=None), 1, "cache is NULL"),
    (dict(cache=FAKE + 8), 3, "cache"),
    (dict(sinv=None), 1, "scale_inv is NULL"),
    (dict(sinv=FAKE + 2), 3, "scale_inv"),
    (dict(in_dt=4), 1, "in_dtype"),
    (dict(flags=2), 1, "flag"),
    (dict(ld=1000), 1, "ld="),
    (dict(ld=1028), 3, "multiple of 8"),
    (dict(x=None), 1, "x is NULL"),
    (dict(x=FAKE + 8), 3, "x must be"),
    (dict(slots=FAKE + 4), 3, "slots"),
    (dict(diag=FAKE + 2), 3, "diag"),
])
def test_kv_store_validation(kw, status, needle):
    st, msg = kvs(**kw)
    assert st == status, (st, msg)
    assert needle in msg


def test_kv_store_bf16_needs_no_scales():
    """BF16 storage ignores scale_inv: NULL passes validation, which then stops
    at the device check (no GPU here) or at a later argument."""
    st, msg = kvs(storage=L.FP8_KV_BF16, sinv=None, x=None)
    assert st == 1 and "x is NULL" in msg


def kvl(**kw):
    a = dict(cache=FAKE, storage=L.FP8_KV_E4M3, scaling=L.FP8_KV_PER_HEAD, sinv=FAKE, cap=64, heads=8, hd=128,
             slots=None, n=16, out_dt=L.FP8_OUT_BF16, out=FAKE, ld_out=1024)
    a.update(kw)
    st = L.lib().fp8_kv_load(a["cache"], a["storage"], a["scaling"], a["sinv"], a["cap"], a["heads"], a["hd"],
                             a["slots"], a["n"], a["out_dt"], a["out"], a["ld_out"], None)
    return st, L.lib().fp8_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(storage=-1), 1, "storage"),
    (dict(hd=12), 2, "head_dim"),
    (dict(sinv=None), 1, "scale_inv is NULL"),
    (dict(out_dt=2), 1, "out_dtype"),
    (dict(ld_out=512), 1, "ld_out="),
    (dict(ld_out=1025), 3, "multiple of 8"),
    (dict(out=None), 1, "out is NULL"),
    (dict(out=FAKE + 4), 3, "out must be"),
    (dict(slots=FAKE + 1), 3, "slots"),
])
def test_kv_load_validation(kw, status, needle):
    st, msg = kvl(**kw)
    assert st == status, (st, msg)
    assert needle in msg


def gemm(**kw):
    a = dict(A=FAKE, fa=0, lda=256, B=FAKE, fb=0, ldb=256, M=256, N=256, K=256, sa=FAKE, ar=0,
             sb=FAKE, br=0, C=FAKE, out=L.FP8_OUT_BF16, ldc=256)
    a.update(kw)
    st = L.lib().fp8_scaled_gemm(a["A"], a["fa"], a["lda"], a["B"], a["fb"], a["ldb"], a["M"], a["N"],
                                 a["K"], a["sa"], a["ar"], a["sb"], a["br"], a["C"], a["out"], a["ldc"],
                                 None)
    return st, L.lib().fp8_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(fa=2), 1, "formats"),
    (dict(ar=2), 1, "per_row"),
    (dict(A=None), 1, "NULL"),
    (dict(C=None), 1, "C is NULL"),
    (dict(sa=None), 1, "scale"),
    (dict(out=5), 1, "out_dtype"),
    (dict(M=-1), 1, "negative"),
    (dict(K=200, lda=256, ldb=256), 2, "multiple of 16"),
    (dict(lda=128), 1, "lda"),
    (dict(ldc=100), 1, "ldc"),
    (dict(A=FAKE + 8), 3, "16-byte"),
    (dict(lda=272 + 8), 3, "multiples of 16"),
    (dict(C=FAKE + 1), 3, "C is not aligned"),
    (dict(out=L.FP8_OUT_F32, C=FAKE + 2), 3, "C is not aligned"),
    (dict(M=2 ** 31), 2, "2^31"),
])
def test_gemm_validation(kw, status, needle):
    st, msg = gemm(**kw)
    assert st == status, (st, msg)
    assert needle in msg


def test_blockgemm_validation():
    lib = L.lib()
    for (M, N, K), needle in [((256, 200, 256), "N % 128"), ((256, 256, 192), "K % 128"),
                              ((256, 256, 0), "K > 0")]:
        st = lib.fp8_blockscaled_gemm(FAKE, 256, FAKE, 256, M, N, K, FAKE, FAKE, FAKE, 1, 256, None)
        assert st == L.FP8_ERR_UNSUPPORTED_SHAPE
        assert needle.split()[0] in lib.fp8_last_error().decode()


def test_history_and_amax_validation():
    lib = L.lib()
    assert lib.fp8_history_set_guard(None, 10.0, None) == L.FP8_ERR_INVALID_ARG
    assert lib.fp8_history_set_guard(FAKE + 4, 10.0, None) == L.FP8_ERR_MISALIGNED
    assert lib.fp8_history_init(None, 16, None) == L.FP8_ERR_INVALID_ARG
    assert lib.fp8_history_init(FAKE, 0, None) == L.FP8_ERR_INVALID_ARG
    assert lib.fp8_history_init(FAKE, 17, None) == L.FP8_ERR_INVALID_ARG
    assert lib.fp8_history_init(FAKE + 8, 16, None) == L.FP8_ERR_MISALIGNED
    W = L.WORKSPACE_BYTES
    assert lib.fp8_amax(FAKE, 1, 4, 4, 4, 5, FAKE, FAKE, W, None) == L.FP8_ERR_INVALID_ARG
    assert lib.fp8_amax(FAKE, 1, 4, 4, 4, 0, None, FAKE, W, None) == L.FP8_ERR_INVALID_ARG
    assert lib.fp8_amax(FAKE + 1, 1, 4, 4, 4, 0, FAKE, FAKE, W, None) == L.FP8_ERR_MISALIGNED
    assert lib.fp8_amax(FAKE, 1, 4, 4, 4, 0, FAKE, None, W, None) == L.FP8_ERR_INVALID_ARG
    assert "workspace" in lib.fp8_last_error().decode()


def test_history_struct_is_128_bytes():
    text = open(L.HEADER).read()
    body = text[text.index("typedef struct fp8_amax_history"):]
    body = body[:body.index("} fp8_amax_history;")]
    # amax, len/pos/count, internal, scale pair, steps, spike threshold, spikes, sync, reserved
    words = 16 + 3 + 2 + 2 + 1 + 1 + 1 + 3 + 3
    assert "float amax[16]" in body and "uint32_t internal[2]" in body and "uint32_t sync[3]" in body
    assert "uint32_t reserved[3]" in body
    assert "float spike_threshold" in body and "uint32_t spikes" in body
    assert words * 4 == L.HISTORY_BYTES


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(ImportError):
        L.lib()


def test_probe_library_exports_its_header():
    """libfp8probe.so (the benchmark's HBM streaming probes) exports what
    include/fp8probe.h declares and nothing of the FP8 method."""
    import re
    probe = os.path.join(os.path.dirname(L.LIB_PATH), "libfp8probe.so")
    text = open(os.path.join(os.path.dirname(L.HEADER), "fp8probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    declared = set(re.findall(r"\b(fp8probe_[a-z_0-9]+)\s*\(", text))
    out = subprocess.run(["nm", "-D", "--defined-only", probe], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert declared == {"fp8probe_read", "fp8probe_copy", "fp8probe_read2_write1"}
    assert declared <= exported and not any(s.startswith("fp8_") for s in exported)
    lib = ctypes.CDLL(probe)
    lib.fp8probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    assert lib.fp8probe_copy(FAKE, FAKE, 24, 4, None) == -1      # not a multiple of 16: nothing launched
