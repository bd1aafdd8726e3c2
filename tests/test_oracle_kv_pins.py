"""Pins of the oracle's FP8 KV cache (or_kv_store / or_kv_load) against
numpy, torch's float8 / bfloat16 CPU casts (library routines), the format's
rounding bound and invariants of the scatter/gather.

Page: "DeepL bets on FP8" (hmyw.cn), section 3.1 (FP8 KV cache; one layer's
K cache kept in BF16).  The layout and scale granularities are readings
stated in the oracle source (O9)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.test_oracle_pins import TORCH_DT, torch_sat_encode

FMTS = {"e4m3": oracle.E4M3, "e5m2": oracle.E5M2}


def _kv_input(n, heads, hd, seed, spread=True):
    """Per-(token, head) magnitudes spread over several binades, so that a
    scale taken from the wrong group changes codes."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(4, size=(n, heads, hd)).astype(np.float32)
    if spread:
        x *= (2.0 ** rng.uniform(-6, 6, size=(n, heads, 1))).astype(np.float32)
    return x.reshape(n, heads * hd)


def _empty_cache(capacity, heads, hd, storage):
    dt = np.uint16 if storage == "bf16" else np.uint8
    return np.zeros((capacity, heads, hd), dtype=dt), np.zeros((capacity, heads), dtype=np.float32)


@pytest.mark.parametrize("storage", ["e4m3", "e5m2"])
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("in_bf16", [False, True])
def test_kv_store_token_head_vs_numpy_torch(storage, pow2, in_bf16):
    n, heads, hd = 37, 3, 96
    xf = _kv_input(n, heads, hd, 1)
    x = synth.to_bf16_bits(xf) if in_bf16 else xf
    xv = synth.bf16_bits_to_f32(x) if in_bf16 else xf
    cache, si = _empty_cache(n, heads, hd, storage)
    c = oracle.kv_store(x, heads, hd, cache, si, storage, "token_head", pow2=pow2)
    fmt = FMTS[storage]
    fmax = np.float32(oracle.format_max(fmt))
    x3 = xv.reshape(n, heads, hd)
    am = np.abs(x3).max(axis=2)
    s = (fmax / am).astype(np.float32)
    if pow2:
        s = np.float32(2.0) ** (np.frexp(s)[1] - 1).astype(np.float32)
    assert np.array_equal(si, (np.float32(1) / s).astype(np.float32))
    prod = (x3 * s[:, :, None]).astype(np.float32)
    assert np.array_equal(cache, torch_sat_encode(fmt, prod))
    # fl32(fmax / amax) * amax may round one ulp above fmax: counted, code = max
    assert c["sat"] == int((np.abs(prod) > fmax).sum())


@pytest.mark.parametrize("storage", ["e4m3", "e5m2"])
def test_kv_store_per_head_static_scale(storage):
    """Given per-head scale_inv (powers of two, one deliberately too small):
    codes = saturating RNE of x / scale_inv, and the saturation counter counts
    exactly the products beyond the format's maximum."""
    n, heads, hd = 50, 4, 64
    xf = _kv_input(n, heads, hd, 2, spread=False)
    fmt = FMTS[storage]
    fmax = np.float32(oracle.format_max(fmt))
    si = np.float32([2.0 ** -4, 2.0 ** -6, 2.0 ** 2, 1.0]) * (1 if storage == "e4m3" else 2.0 ** -7)
    si = si.astype(np.float32)
    cache, _ = _empty_cache(n, heads, hd, storage)
    c = oracle.kv_store(xf, heads, hd, cache, si, storage, "head")
    prod = (xf.reshape(n, heads, hd) / si[None, :, None]).astype(np.float32)
    assert np.array_equal(cache, torch_sat_encode(fmt, prod))
    nsat = int((np.abs(prod) > fmax).sum())
    assert nsat > 0 and c["sat"] == nsat


@pytest.mark.parametrize("storage", ["e4m3", "e5m2"])
@pytest.mark.parametrize("scaling", ["token_head", "head"])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_kv_load_vs_torch_decode(storage, scaling, out_bf16):
    """y = fl32(decode(q) * scale_inv) over all 256 codes, then bf16 RNE."""
    heads, hd, n = 2, 128, 40
    fmt = FMTS[storage]
    rng = np.random.default_rng(3)
    cache = rng.integers(0, 256, size=(n, heads, hd), dtype=np.uint8)
    cache[0, 0, :] = np.arange(128, dtype=np.uint8)
    cache[0, 1, :] = np.arange(128, 256, dtype=np.uint8)
    if scaling == "token_head":
        si = (2.0 ** rng.uniform(-12, 4, size=(n, heads))).astype(np.float32)
        sfull = si[:, :, None]
    else:
        si = np.float32([0.37, 3.1e-3])
        sfull = si[None, :, None]
    y = oracle.kv_load(cache, si, n, storage, scaling, out_bf16=out_bf16)
    dec = torch.from_numpy(cache).view(TORCH_DT[fmt]).to(torch.float32)
    ref = dec * torch.from_numpy(np.ascontiguousarray(np.broadcast_to(sfull, cache.shape)))
    if out_bf16:
        ref = ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).reshape(n, -1)
        nan = np.isnan(synth.bf16_bits_to_f32(ref))
        assert np.array_equal(np.isnan(synth.bf16_bits_to_f32(y)), nan)
        assert np.array_equal(y[~nan], ref[~nan])
    else:
        ref = ref.numpy().reshape(n, -1)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(y), nan)
        assert np.array_equal(y[~nan], ref[~nan])


def test_kv_bf16_storage_is_torch_rounding():
    """The BF16 fallback layer: fp32 input rounded by torch's RNE cast; bf16
    input stored bit for bit; load returns the stored values."""
    n, heads, hd = 21, 2, 64
    xf = _kv_input(n, heads, hd, 4)
    cache, si = _empty_cache(n, heads, hd, "bf16")
    oracle.kv_store(xf, heads, hd, cache, si, "bf16")
    ref = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(cache.reshape(n, -1), ref)
    assert not si.any()
    xb = synth.to_bf16_bits(xf)
    cache2, _ = _empty_cache(n, heads, hd, "bf16")
    oracle.kv_store(xb, heads, hd, cache2, si, "bf16")
    assert np.array_equal(cache2.reshape(n, -1), xb)
    assert np.array_equal(oracle.kv_load(cache2, si, n, "bf16"), xb)
    y32 = oracle.kv_load(cache2, si, n, "bf16", out_bf16=False)
    assert np.array_equal(y32, synth.bf16_bits_to_f32(xb))


@pytest.mark.parametrize("storage", ["e4m3", "e5m2"])
def test_kv_roundtrip_within_half_ulp(storage):
    """load(store(x)) in fp32: |y - x| <= 2^-(m+1) |x| for values in the
    normal range of the scaled format, and <= half the subnormal spacing
    times scale_inv below it (m = mantissa bits)."""
    n, heads, hd = 64, 4, 128
    x = _kv_input(n, heads, hd, 5)
    cache, si = _empty_cache(n, heads, hd, storage)
    oracle.kv_store(x, heads, hd, cache, si, storage)
    y = oracle.kv_load(cache, si, n, storage, out_bf16=False)
    m, emin_sub = (3, -9) if storage == "e4m3" else (2, -16)
    sfull = np.repeat(si, hd, axis=1)
    bound = np.maximum(np.abs(x) * 2.0 ** -(m + 1), sfull * 2.0 ** (emin_sub - 1)) * (1 + 2 ** -20)
    assert (np.abs(y.astype(np.float64) - x) <= bound).all()
    # the largest element of each (token, head) lands on the format's maximum
    x3 = np.abs(x.reshape(n, heads, hd))
    i = x3.argmax(axis=2)
    top = np.take_along_axis(cache, i[:, :, None], axis=2)[:, :, 0] & 0x7F
    assert (top == (0x7E if storage == "e4m3" else 0x7B)).all()


def test_kv_slots_scatter_gather_invariants():
    """Scatter by a permutation with padding, gather by the same slots:
    equal to the contiguous store row for row; padded tokens write nothing
    and leave their output rows untouched; rows never written stay zero."""
    n, heads, hd, cap = 30, 2, 64, 48
    x = _kv_input(n, heads, hd, 6)
    c0, s0 = _empty_cache(n, heads, hd, "e4m3")
    oracle.kv_store(x, heads, hd, c0, s0)
    rng = np.random.default_rng(8)
    slots = rng.permutation(cap)[:n].astype(np.int64)
    slots[[4, 17]] = -1
    slots[9] = cap + 3                           # outside the cache: not stored
    c1, s1 = _empty_cache(cap, heads, hd, "e4m3")
    oracle.kv_store(x, heads, hd, c1, s1, slots=slots)
    ok = (slots >= 0) & (slots < cap)
    assert np.array_equal(c1[slots[ok]], c0[ok]) and np.array_equal(s1[slots[ok]], s0[ok])
    untouched = np.setdiff1d(np.arange(cap), slots[ok])
    assert not c1[untouched].any() and not s1[untouched].any()
    sentinel = np.full((n, heads * hd), 0xABCD, dtype=np.uint16)
    y = oracle.kv_load(c1, s1, n, slots=slots, out=sentinel)
    ref = oracle.kv_load(c0, s0, n)
    assert np.array_equal(y[ok], ref[ok])
    assert (y[~ok] == 0xABCD).all()


def test_kv_store_nonfinite_and_zero_rows():
    """A NaN element makes its (token, head) amax non-finite -> s = 1 (O4)
    and the NaN keeps a NaN code; an Inf saturates; an all-zero vector gets
    s = 1 and zero codes; other heads are unaffected."""
    n, heads, hd = 4, 3, 64
    x = _kv_input(n, heads, hd, 9)
    x3 = x.reshape(n, heads, hd)
    x3[1, 0, 5] = np.nan
    x3[2, 2, 7] = np.inf
    x3[3, 1, :] = 0.0
    cache, si = _empty_cache(n, heads, hd, "e4m3")
    c = oracle.kv_store(x, heads, hd, cache, si)
    assert si[1, 0] == 1 and si[2, 2] == 1 and si[3, 1] == 1
    assert cache[1, 0, 5] & 0x7F == 0x7F
    assert cache[2, 2, 7] == 0x7E
    assert not cache[3, 1].any()
    assert c["nonfinite"] == 2
    ref, _ = _empty_cache(n, heads, hd, "e4m3")
    ref_si = np.zeros_like(si)
    clean = x.copy().reshape(n, heads, hd)
    oracle.kv_store(clean.reshape(n, -1), heads, hd, ref, ref_si)
    assert np.array_equal(ref[0], cache[0]) and np.array_equal(ref_si[0], si[0])
