"""The binding's buffer checks (host logic, no GPU): a buffer the library
would read or write as n packed elements must have that many, be
contiguous, have the dtype and sit on the device of the call; an output
matrix must have its shape and a contiguous last dimension."""
from __future__ import annotations

import pytest
import torch

fp8 = pytest.importorskip("fp8_precision_quantization_amd")

CPU = torch.device("cpu")


def test_buf_accepts_exact_buffers():
    t = torch.zeros((4, 3), dtype=torch.float32)
    assert fp8._buf(t, 12, torch.float32, CPU, "s") == t.data_ptr()
    assert fp8._buf(torch.zeros(1), 1, torch.float32, CPU, "s") != 0


@pytest.mark.parametrize("t, n, dtype, exc, msg", [
    (torch.zeros(11), 12, torch.float32, ValueError, "of 12 elements"),
    (torch.zeros((4, 6))[:, ::2], 12, torch.float32, ValueError, "contiguous"),
    (torch.zeros(12, dtype=torch.float64), 12, torch.float32, TypeError, "torch.float32"),
    (torch.zeros(12, dtype=torch.int32), 12, torch.float32, TypeError, "got torch.int32"),
])
def test_buf_rejects(t, n, dtype, exc, msg):
    with pytest.raises(exc, match=msg):
        fp8._buf(t, n, dtype, CPU, "s")


def test_buf_rejects_other_device():
    with pytest.raises(ValueError, match="must be a tensor on"):
        fp8._buf(torch.zeros(4), 4, torch.float32, torch.device("cuda", 0), "s")
    with pytest.raises(ValueError, match="must be a tensor on"):
        fp8._buf(None, 4, torch.float32, CPU, "s")


def test_out_matrix_leading_dimension():
    full = torch.zeros((8, 40), dtype=torch.uint8)
    assert fp8._out_matrix(full, 8, 40, torch.uint8, CPU, "out") == 40
    assert fp8._out_matrix(full[:, :33], 8, 33, torch.uint8, CPU, "out") == 40    # a view with a row pitch
    assert fp8._out_matrix(torch.zeros((1, 5), dtype=torch.uint8), 1, 5, torch.uint8, CPU, "out") == 5


@pytest.mark.parametrize("out, shape, dtype, exc, msg", [
    (torch.zeros((8, 40), dtype=torch.uint8), (8, 39), torch.uint8, ValueError, "must have shape"),
    (torch.zeros((8, 40), dtype=torch.uint8), (40, 8), torch.uint8, ValueError, "must have shape"),
    (torch.zeros((8, 40), dtype=torch.int8), (8, 40), torch.uint8, TypeError, "must be torch.uint8"),
    (torch.zeros((40, 8), dtype=torch.uint8).t(), (8, 40), torch.uint8, ValueError, "contiguous last dimension"),
])
def test_out_matrix_rejects(out, shape, dtype, exc, msg):
    with pytest.raises(exc, match=msg):
        fp8._out_matrix(out, shape[0], shape[1], dtype, CPU, "out")


@pytest.mark.parametrize("storage, scaling, capacity, heads, n", [
    ("e4m3", "token_head", 16, 2, 32), ("e5m2", "head", 16, 2, 2)])
def test_kv_scales_sizes(storage, scaling, capacity, heads, n):
    ok = torch.zeros(n)
    assert fp8._kv_scales(ok, storage, scaling, capacity, heads, CPU) == ok.data_ptr()
    with pytest.raises(ValueError, match="of %d elements" % n):
        fp8._kv_scales(torch.zeros(n + 1), storage, scaling, capacity, heads, CPU)
    # bf16 storage has no scales: whatever is passed goes through unchecked
    assert fp8._kv_scales(None, "bf16", scaling, capacity, heads, CPU) is None
