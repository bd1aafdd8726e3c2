"""Host logic of the KV-cache binding that needs no GPU: the per-layer
storage choice (BF16 fallback layers) and the memory it takes, on CPU
tensors (no kernel is called)."""
from __future__ import annotations

import pytest
import torch

fp8 = pytest.importorskip("fp8_precision_quantization_amd")


def test_kv_cache_memory_halves():
    """[DeepL] 3.1: FP8 storage holds a layer's K/V in about half the bytes
    of bf16 (the per-(token, head) scales add 4 bytes per head_dim values)."""
    H, D, cap = 8, 128, 4096
    a = fp8.KVCache(4, cap, H, D, device="cpu")
    b = fp8.KVCache(4, cap, H, D, storage="bf16", device="cpu")
    c = fp8.KVCache(4, cap, H, D, bf16_k_layers=[3], device="cpu")
    assert b.nbytes == 4 * 2 * cap * H * D * 2
    assert a.nbytes == 4 * 2 * (cap * H * D + cap * H * 4)
    assert abs(a.nbytes / b.nbytes - (0.5 + 2 / D)) < 1e-12
    assert c.nbytes == a.nbytes + cap * H * D - cap * H * 4


def test_kv_fallback_layers_and_scale_shapes():
    c = fp8.KVCache(3, 64, 2, 64, bf16_k_layers=[1], bf16_v_layers=[2], device="cpu")
    assert [t.data.dtype for t in c.k] == [torch.uint8, torch.bfloat16, torch.uint8]
    assert [t.data.dtype for t in c.v] == [torch.uint8, torch.uint8, torch.bfloat16]
    assert c.k[0].scale_inv.shape == (64, 2) and c.k[1].scale_inv is None
    hs = torch.tensor([[[0.5, 0.25]] * 3, [[1.0, 2.0]] * 3])
    d = fp8.KVCache(3, 64, 2, 64, scaling="head", head_scale_inv=hs, device="cpu")
    assert d.k[2].scale_inv.tolist() == [0.5, 0.25] and d.v[0].scale_inv.tolist() == [1.0, 2.0]
    with pytest.raises(ValueError):
        fp8.KVCache(2, 8, 1, 64, bf16_k_layers=[2], device="cpu")
    with pytest.raises(ValueError):
        fp8.KVTensorCache(8, 2, 64, scaling="head", device="cpu")
    with pytest.raises(ValueError):
        fp8.kv_store(torch.zeros(4, 128), c.k[0].data, c.k[0].scale_inv)   # host tensor
