"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- the page constants (tests/golden/page_facts.txt), torch's
float8_e4m3fn / float8_e5m2 / bfloat16 CPU casts (library routines), numpy,
exact integer or rational arithmetic, and brute force on tiny inputs.  A
plausible mistake anywhere in the oracle (a dropped term, a wrong sign, an
off-by-one in the ring, a transposed operand) fails at least one of them.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import check_gemm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.txt")
TORCH_DT = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}
FMTS = [oracle.E4M3, oracle.E5M2]


def page_facts():
    facts = {}
    with open(GOLDEN) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            key, val, src = [s.strip() for s in line.split("|")]
            facts[key] = (val, src)
    return facts


def torch_decode(fmt) -> np.ndarray:
    codes = torch.arange(256, dtype=torch.uint8)
    return codes.view(TORCH_DT[fmt]).to(torch.float64).numpy()


def torch_sat_encode(fmt, v: np.ndarray) -> np.ndarray:
    """Library-routine pin: torch's cast is RNE but not saturating, so clamp to
    +-max first (identical to saturating RNE for every non-NaN input)."""
    fmax = torch.finfo(TORCH_DT[fmt]).max
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    t = t.clamp(-fmax, fmax)
    return t.to(TORCH_DT[fmt]).view(torch.uint8).numpy()


# ------------------------------------------------------------------ decode --
@pytest.mark.parametrize("fmt", FMTS)
def test_decode_matches_torch(fmt):
    ours = oracle.decode_table(fmt)
    ref = torch_decode(fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_decode_page_constants():
    facts = page_facts()
    e5m2_range = float(facts["e5m2_range"][0])
    t5 = oracle.decode_table(oracle.E5M2)
    fin5 = t5[np.isfinite(t5)]
    assert fin5.max() == e5m2_range and fin5.min() == -e5m2_range
    assert oracle.format_max(oracle.E5M2) == e5m2_range
    # bit splits: the number of distinct positive normal binades is 2^e - 2 (E5M2,
    # IEEE-style top exponent reserved) and 2^e - 1 (E4M3, only S.1111.111 is
    # NaN); every binade holds 2^m values.
    for fmt, key in ((oracle.E4M3, "e4m3_bits"), (oracle.E5M2, "e5m2_bits")):
        spec = dict(kv.split("=") for kv in facts[key][0].split())
        e, m = int(spec["exponent"]), int(spec["mantissa"])
        assert int(spec["sign"]) + e + m == 8
        t = oracle.decode_table(fmt)
        pos = t[:128]
        normals = pos[np.isfinite(pos) & (pos >= pos[1 << m])]
        binades = np.unique(np.floor(np.log2(normals)))
        expect = (2 ** e - 1) if fmt == oracle.E4M3 else (2 ** e - 2)
        assert binades.size == expect
        counts = [int(np.sum(np.floor(np.log2(normals)) == b)) for b in binades]
        # every binade holds 2^m values; E4M3's top binade gives one up to NaN
        top_loss = 1 if fmt == oracle.E4M3 else 0
        assert counts[:-1] == [2 ** m] * (len(counts) - 1)
        assert counts[-1] == 2 ** m - top_loss
    # E4M3: smaller range, finer mantissa than E5M2
    t4 = oracle.decode_table(oracle.E4M3)
    assert np.nanmax(t4) < fin5.max()
    assert t4[0x39] - t4[0x38] < t5[0x3D] - t5[0x3C]   # spacing just above 1.0


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_sign_symmetry_and_monotone(fmt):
    t = oracle.decode_table(fmt)
    pos, neg = t[:128], t[128:]
    fin = np.isfinite(pos) & np.isfinite(neg)
    assert np.array_equal(-pos[fin], neg[fin])
    p = pos[np.isfinite(pos)]
    assert np.all(np.diff(p) > 0)


# ------------------------------------------------------------------ encode --
@pytest.mark.parametrize("fmt", FMTS)
def test_encode_all_bf16_patterns(fmt):
    bits = np.arange(65536, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    assert np.array_equal(oracle.encode(fmt, v), torch_sat_encode(fmt, v))


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_midpoints_and_neighbours(fmt):
    t = oracle.decode_table(fmt)
    pos = t[:128]
    pos = pos[np.isfinite(pos)].astype(np.float32)
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1].astype(np.float64) + pos[1:]) / 2)
    cand = [mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
            pos, np.nextafter(pos, np.float32(np.inf)), np.nextafter(pos, np.float32(0))]
    fmax = np.float32(pos.max())
    cand.append(np.array([fmax, np.nextafter(fmax, np.float32(np.inf)), fmax * 1.03125,
                          fmax * 1.0625, fmax * 2, np.float32(3.0e38), np.inf], np.float32))
    v = np.concatenate(cand)
    v = np.concatenate([v, -v])
    assert np.array_equal(oracle.encode(fmt, v), torch_sat_encode(fmt, v))


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_ties_go_to_even_code(fmt):
    t = oracle.decode_table(fmt)
    pos = t[:128]
    n = int(np.isfinite(pos).sum())
    for c in range(n - 1):
        mid = np.float32((pos[c] + pos[c + 1]) / 2)
        code = int(oracle.encode(fmt, np.array([mid]))[0])
        assert code in (c, c + 1) and code % 2 == 0


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_random_and_strided_fp32(fmt):
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # strided sweep through the whole binary32 space
    bits = np.concatenate([bits, (np.arange(0, 2 ** 32, 2039, dtype=np.uint64)).astype(np.uint32)])
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    assert np.array_equal(oracle.encode(fmt, v), torch_sat_encode(fmt, v))


def active_binades(fmt):
    """Unbiased exponents e whose binade [2^e, 2^(e+1)) holds fp32 values
    with more than one FP8 code: from two binades below the smallest
    subnormal to the binade past the largest finite value.  Every fp32
    below encodes to +-0 and every one above saturates."""
    t = oracle.decode_table(fmt)
    pos = t[:128][np.isfinite(t[:128])]
    lo = int(np.floor(np.log2(pos[pos > 0].min()))) - 2
    hi = int(np.ceil(np.log2(pos.max()))) + 1
    return range(lo, hi)


def binade_bits(e: int, sign: int) -> np.ndarray:
    return (np.uint32(sign << 31) | np.uint32((e + 127) << 23) |
            np.arange(1 << 23, dtype=np.uint32)).astype(np.uint32)


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_exhaustive_over_active_binades(fmt):
    """Every fp32 of both signs in the binades where the code varies (E4M3:
    21 binades, E5M2: 35; 2^23 values each) against torch's clamped cast;
    the binades outside are covered by the strided sweep above."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = [(e, sg) for e in active_binades(fmt) for sg in (0, 1)]

    def check(job):
        v = binade_bits(*job).view(np.float32)
        return job, np.array_equal(oracle.encode(fmt, v), torch_sat_encode(fmt, v))

    with ThreadPoolExecutor(max_workers=8) as ex:
        bad = [job for job, ok in ex.map(check, jobs) if not ok]
    assert not bad, bad
    assert len(jobs) == 2 * (21 if fmt == oracle.E4M3 else 35)


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_specials(fmt):
    top = 0x7E if fmt == oracle.E4M3 else 0x7B
    v = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, -1e-30, 1e-30], np.float32)
    v[1] = np.float32(-np.nan) if np.signbit(np.float32(-np.nan)) else -np.abs(v[0])
    codes = oracle.encode(fmt, v).tolist()
    assert codes[0] == 0x7F and codes[1] == 0xFF            # NaN keeps its sign
    assert codes[2] == top and codes[3] == 0x80 | top        # saturating
    assert codes[4] == 0x00 and codes[5] == 0x80
    assert codes[6] == 0x80 and codes[7] == 0x00             # sign kept on underflow


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_decode_roundtrip(fmt):
    t = oracle.decode_table(fmt)
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], np.uint8)
    back = oracle.encode(fmt, t[codes].astype(np.float32))
    assert np.array_equal(back, codes)


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_monotone(fmt):
    rng = np.random.default_rng(5)
    v = np.sort(rng.standard_normal(200_000).astype(np.float32) * 300)
    t = oracle.decode_table(fmt)
    vals = t[oracle.encode(fmt, v)]
    assert np.all(np.diff(vals) >= 0)


# ------------------------------------------------------------ amax / scale --
def test_amax_matches_numpy_all_granularities():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((300, 515)).astype(np.float32) * 3
    a = np.abs(x)
    assert oracle.amax(x, "tensor")[0, 0] == a.max()
    assert np.array_equal(oracle.amax(x, "row")[:, 0], a.max(axis=1))
    blk = oracle.amax(x, "1x128")
    for kb in range(5):
        assert np.array_equal(blk[:, kb], a[:, kb * 128:(kb + 1) * 128].max(axis=1))
    b2 = oracle.amax(x, "128x128")
    assert b2.shape == (3, 5)
    for rb in range(3):
        for kb in range(5):
            assert b2[rb, kb] == a[rb * 128:(rb + 1) * 128, kb * 128:(kb + 1) * 128].max()
    xb = synth.to_bf16_bits(x)
    assert oracle.amax(xb, "tensor")[0, 0] == np.abs(synth.bf16_bits_to_f32(xb)).max()


def test_amax_nonfinite():
    x = np.ones((4, 8), np.float32)
    x[1, 2] = np.inf
    assert np.isinf(oracle.amax(x)[0, 0])
    x[3, 3] = np.nan
    assert np.isnan(oracle.amax(x)[0, 0])
    assert np.isinf(oracle.amax(x, "row")[1, 0]) and np.isnan(oracle.amax(x, "row")[3, 0])


@pytest.mark.parametrize("fmt", FMTS)
def test_scale_matches_numpy_division(fmt):
    rng = np.random.default_rng(1)
    fmax = np.float32(oracle.format_max(fmt))
    for a in np.concatenate([rng.random(500).astype(np.float32) * 1e3,
                             np.float32([1e-38, 1e-45, 3e38, 448, 57344, 1])]):
        s, si = oracle.scale(a, fmt)
        with np.errstate(over="ignore"):
            ref = np.float32(fmax / np.float32(a))
        if np.isinf(ref):
            ref = np.finfo(np.float32).max
        assert s == ref
        assert si == np.float32(np.float32(1) / ref)
    for a in [0.0, np.inf, np.nan]:
        s, si = oracle.scale(a, fmt)
        assert s == 1.0 and si == 1.0


@pytest.mark.parametrize("fmt", FMTS)
def test_scale_pow2_is_floor_power_of_two(fmt):
    rng = np.random.default_rng(2)
    fmax = np.float32(oracle.format_max(fmt))
    for a in rng.random(500).astype(np.float32) * 100 + 1e-3:
        s, si = oracle.scale(a, fmt, pow2=True)
        q = float(np.float32(fmax / a))
        mant, ex = np.frexp(q)                 # q = mant * 2^ex, mant in [0.5, 1)
        assert float(s) == 2.0 ** (ex - 1)
        assert float(si) * float(s) == 1.0       # exact reciprocal
    s, _ = oracle.scale(1e-45, fmt, pow2=True)
    assert float(s) == 2.0 ** 127


# -------------------------------------------------------------- quantize --
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("gran", ["tensor", "row", "1x128", "128x128"])
@pytest.mark.parametrize("pow2", [False, True])
def test_quantize_composition_vs_torch(fmt, gran, pow2):
    rng = np.random.default_rng(7)
    rows, cols = 260, 390
    x = rng.standard_t(3, size=(rows, cols)).astype(np.float32) * 2
    x[5, :] = 0.0                               # an all-zero row -> s = 1
    xb = synth.to_bf16_bits(x)
    xf = synth.bf16_bits_to_f32(xb)
    r = oracle.quantize(xb, fmt, gran, pow2)
    # expected from numpy + torch only
    h, w = {"tensor": (rows, cols), "row": (1, cols), "1x128": (1, 128),
            "128x128": (128, 128)}[gran]
    gr, gc = -(-rows // h), -(-cols // w)
    fmax = np.float32(oracle.format_max(fmt))
    s_full = np.empty_like(xf)
    for i in range(gr):
        for j in range(gc):
            blk = np.abs(xf[i * h:(i + 1) * h, j * w:(j + 1) * w])
            am = blk.max()
            assert r["amax"].reshape(gr, gc)[i, j] == am
            s = np.float32(1.0) if am == 0 else np.float32(fmax / am)
            if pow2:
                s = np.float32(2.0 ** (np.frexp(float(s))[1] - 1))
            assert r["scale"].reshape(gr, gc)[i, j] == s
            s_full[i * h:(i + 1) * h, j * w:(j + 1) * w] = s
    prod = (xf * s_full).astype(np.float32)
    assert np.array_equal(r["q"], torch_sat_encode(fmt, prod))
    assert r["sat"] == int((np.abs(prod) > fmax).sum())
    t = oracle.decode_table(fmt)
    under = int(((xf != 0) & (t[r["q"]] == 0)).sum())
    assert r["underflow"] == under


def test_quantize_counts_nonfinite():
    x = np.ones((3, 5), np.float32)
    x[0, 0], x[1, 1], x[2, 2] = np.nan, np.inf, -np.inf
    r = oracle.quantize(x, oracle.E4M3, "row")
    assert r["nonfinite"] == 3
    assert r["q"][0, 0] == 0x7F and r["q"][1, 1] == 0x7E and r["q"][2, 2] == 0xFE
    # rows holding a non-finite amax fall back to s = 1
    assert r["scale"][0, 0] == 1.0 and r["scale"][1, 0] == 1.0


# ---------------------------------------------------------------- delayed --
def _planted(rng, amax_value, shape=(64, 96)):
    x = rng.uniform(-0.5, 0.5, size=shape).astype(np.float32) * amax_value
    x[3, 7] = -amax_value                        # the planted maximum
    return x


@pytest.mark.parametrize("length", [16, 4])
def test_delayed_ring_window_closed_form(length):
    """Planted amaxes a_t: step t must use fl32(fmax / max(a_{t-L..t-1})),
    or the just-in-time scale at t = 0."""
    rng = np.random.default_rng(11)
    amaxes = np.float32(rng.uniform(0.5, 8.0, size=40))
    amaxes[20] = np.float32(300.0)               # a spike
    ds = oracle.DelayedScaler(oracle.E4M3, length)
    fmax = np.float32(448.0)
    for t, a in enumerate(amaxes):
        x = _planted(rng, a)
        r = ds.step(x)
        basis = a if t == 0 else amaxes[max(0, t - length):t].max()
        assert r["scale"] == np.float32(fmax / basis), t
        assert r["amax"] == a
        assert np.array_equal(r["q"], torch_sat_encode(oracle.E4M3, (x * r["scale"]).astype(np.float32)))
        if t == 20:
            assert r["sat"] > 0                 # the spike saturates
        if 21 <= t < 21 + length:
            assert r["scale"] == np.float32(fmax / np.float32(300.0))
        if t == 21 + length:
            assert r["scale"] != np.float32(fmax / np.float32(300.0))


def test_delayed_spike_small_wgrad_run():
    """The wgrad recipe at a reduced size: the spike step saturates dY and the
    following steps rescale from the spike's amax."""
    ds_dy = oracle.DelayedScaler(oracle.E5M2)
    ds_x = oracle.DelayedScaler(oracle.E4M3)
    res = []
    for t in range(16):
        dy, x = synth.wgrad_step(t, tokens=64, hidden=96, spike_step=12)
        res.append((ds_dy.step(dy), ds_x.step(x)))
    a12 = res[12][0]["amax"]
    assert res[12][0]["sat"] > 0
    for t in range(13, 16):
        assert res[t][0]["scale"] == np.float32(np.float32(57344.0) / a12)
        assert res[t][0]["sat"] == 0
    # X's ring never sees the spike: its scale stays within the N(0,1) range
    for t in range(1, 16):
        assert 448.0 / 8.0 < res[t][1]["scale"] < 448.0 / 2.0


def test_delayed_spike_guard_on_the_wgrad_run():
    """The spike guard ([DeepL bets on FP8] 2.3, recovery from a distribution
    jump) with threshold 10: only dY's step 12 trips it; that step equals the
    independently pinned just-in-time cast of the same tensor (codes, scale,
    saturation count), every other step and the final rings equal the
    unguarded run."""
    plain = (oracle.DelayedScaler(oracle.E5M2), oracle.DelayedScaler(oracle.E4M3))
    guard = (oracle.DelayedScaler(oracle.E5M2, spike_threshold=10.0),
             oracle.DelayedScaler(oracle.E4M3, spike_threshold=10.0))
    for t in range(16):
        dy, x = synth.wgrad_step(t, tokens=64, hidden=96, spike_step=12)
        for k, (inp, fmt) in enumerate([(dy, oracle.E5M2), (x, oracle.E4M3)]):
            a, g = plain[k].step(inp), guard[k].step(inp)
            spike = (k == 0 and t == 12)
            assert g["spiked"] == spike, (t, k)
            assert a["spiked"] is False
            if spike:
                jit = oracle.quantize(inp, fmt, "tensor")
                assert np.array_equal(g["q"], jit["q"])
                assert g["scale_inv"] == jit["scale_inv"].ravel()[0]
                assert g["sat"] == jit["sat"] < a["sat"]
            else:
                assert np.array_equal(g["q"], a["q"]) and g["scale"] == a["scale"]
    for k in range(2):
        assert guard[k].state()["amax"].tolist() == plain[k].state()["amax"].tolist()
        assert guard[k].state()["count"] == plain[k].state()["count"]


def test_delayed_spike_guard_threshold_is_strict():
    """amax > threshold * window max trips the guard; equality, an empty
    window and a threshold <= 0 do not."""
    def step(scaler, m):
        return scaler.step(np.array([[m, -0.5]], np.float32))
    for thr, second, want in [(10.0, 10.0, False), (10.0, np.nextafter(np.float32(10), np.float32(20)), True),
                              (0.0, 1e6, False), (-1.0, 1e6, False), (2.0, 2.5, True)]:
        sc = oracle.DelayedScaler(oracle.E4M3, spike_threshold=thr)
        first = step(sc, 1.0)
        assert first["spiked"] is False                  # empty window
        r = step(sc, np.float32(second))
        assert r["spiked"] == want, (thr, second)
        if want:
            assert r["scale"] == np.float32(np.float32(448.0) / np.float32(second))
        else:
            assert r["scale"] == np.float32(448.0)       # from the window's amax 1.0


# ------------------------------------------------------------------- GEMM --
def _rand_codes(rng, shape, fmt):
    t = oracle.decode_table(fmt)
    finite = np.array([c for c in range(256) if np.isfinite(t[c])], np.uint8)
    return rng.choice(finite, size=shape)


def test_gemm_exact_vs_fractions_bruteforce():
    rng = np.random.default_rng(3)
    M, N, K = 3, 4, 40
    for fa, fb in [(oracle.E4M3, oracle.E4M3), (oracle.E5M2, oracle.E4M3), (oracle.E5M2, oracle.E5M2)]:
        A = _rand_codes(rng, (M, K), fa)
        B = _rand_codes(rng, (N, K), fb)
        sa, sb = np.float32(0.37), np.float32(1.9)
        ta, tb = oracle.decode_table(fa), oracle.decode_table(fb)
        ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        ye = oracle.gemm_exact_sampled(A, fa, B, fb, sa, sb, ms.ravel(), ns.ravel())
        for i, (m, n) in enumerate(zip(ms.ravel(), ns.ravel())):
            d = sum(Fraction(float(ta[A[m, k]])) * Fraction(float(tb[B[n, k]])) for k in range(K))
            ref = float(d * Fraction(float(sa)) * Fraction(float(sb)))
            assert ye[i] == pytest.approx(ref, rel=1e-15, abs=1e-300)


def test_gemm_fp32_oracle_vs_exact_and_numpy():
    rng = np.random.default_rng(4)
    M, N, K = 48, 40, 512
    A = _rand_codes(rng, (M, K), oracle.E4M3)
    B = _rand_codes(rng, (N, K), oracle.E5M2)
    sa = rng.random(M).astype(np.float32) + 0.5
    sb = np.float32(0.0625)
    Y, P = oracle.gemm(A, oracle.E4M3, B, oracle.E5M2, sa, sb)
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ye = oracle.gemm_exact_sampled(A, oracle.E4M3, B, oracle.E5M2, sa, sb, ms.ravel(), ns.ravel())
    ok, rep = check_gemm(Y.ravel(), ye.astype(np.float32), P.ravel(), K, "f32")
    assert ok.all(), rep
    # library routine: float64 matmul of the dequantized operands
    Ad = (oracle.decode_table(oracle.E4M3)[A].astype(np.float32) * sa[:, None]).astype(np.float64)
    Bd = oracle.decode_table(oracle.E5M2)[B].astype(np.float32).astype(np.float64) * float(sb)
    ref = Ad @ Bd.T
    assert np.allclose(Y, ref, rtol=0, atol=1e-4 * np.abs(Ad) .max() * np.abs(Bd).max() * K)
    assert np.allclose(P, np.abs(Ad) @ np.abs(Bd).T, rtol=1e-12)
    # sampled form agrees with the full form bit for bit
    y2, p2 = oracle.gemm_sampled(A, oracle.E4M3, B, oracle.E5M2, sa, sb, ms.ravel(), ns.ravel())
    assert np.array_equal(y2, Y.ravel()) and np.array_equal(p2, P.ravel())


def test_gemm_onehot_decodes_every_code():
    """B one-hot with the code for 1.0: Y[m, n] = decode(A[m, k_n]) exactly."""
    for fmt in FMTS:
        t = oracle.decode_table(fmt)
        finite = [c for c in range(256) if np.isfinite(t[c])]
        K = len(finite)
        A = np.array(finite, np.uint8)[None, :].repeat(2, axis=0)
        one = 0x38 if fmt == oracle.E4M3 else 0x3C
        assert t[one] == 1.0
        B = np.zeros((K, K), np.uint8)
        B[np.arange(K), np.arange(K)] = one
        Y, _ = oracle.gemm(A, fmt, B, fmt, 1.0, 1.0)
        assert np.array_equal(Y[0], t[finite].astype(np.float32))


def test_gemm_detects_a_dropped_term():
    """The tolerance rule is sharp enough to see one missing product."""
    rng = np.random.default_rng(8)
    M, N, K = 16, 16, 256
    X = rng.standard_normal((M, K)).astype(np.float32)
    W = rng.standard_normal((N, K)).astype(np.float32)
    qa = oracle.quantize(X, oracle.E4M3)
    qb = oracle.quantize(W, oracle.E4M3)
    Y, P = oracle.gemm(qa["q"], 0, qb["q"], 0, qa["scale_inv"][0, 0], qb["scale_inv"][0, 0])
    A2 = qa["q"].copy()
    A2[:, 17] = 0                                # drop one k term
    Y2, _ = oracle.gemm(A2, 0, qb["q"], 0, qa["scale_inv"][0, 0], qb["scale_inv"][0, 0])
    ok, _ = check_gemm(Y2, Y, P, K, "f32")
    assert (~ok).mean() > 0.5


def test_blockgemm_vs_numpy_and_exact():
    rng = np.random.default_rng(12)
    M, N, K = 20, 256, 384
    A = _rand_codes(rng, (M, K), oracle.E4M3)
    B = _rand_codes(rng, (N, K), oracle.E4M3)
    a_inv = (rng.random((M, K // 128)) + 0.1).astype(np.float32)
    b_inv = (rng.random((N // 128, K // 128)) * 0.01 + 1e-3).astype(np.float32)
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    y, p = oracle.blockgemm_sampled(A, B, a_inv, b_inv, ms.ravel(), ns.ravel())
    t = oracle.decode_table(oracle.E4M3)
    Ad = t[A].astype(np.float32) * np.repeat(a_inv, 128, axis=1)
    Bd = t[B].astype(np.float32) * np.repeat(np.repeat(b_inv, 128, axis=0), 128, axis=1)
    ref = Ad.astype(np.float64) @ Bd.astype(np.float64).T
    ok, rep = check_gemm(y, ref.ravel().astype(np.float32), p, K, "f32")
    assert ok.all(), rep
    ye = oracle.gemm_exact_sampled(A, 0, B, 0, a_inv, b_inv, ms.ravel(), ns.ravel(), block_mode=True)
    # the exact path does not round the dequantized operands to fp32
    Ad64 = t[A] * np.repeat(a_inv.astype(np.float64), 128, axis=1)
    Bd64 = t[B] * np.repeat(np.repeat(b_inv.astype(np.float64), 128, axis=0), 128, axis=1)
    ref64 = Ad64 @ Bd64.T
    assert np.allclose(ye, ref64.ravel(), rtol=1e-12, atol=1e-12 * np.abs(ref64).max())


# ------------------------------------------------------------- bf16 output --
def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(13)
    bits = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    # exact ties and the overflow boundary
    ties = ((rng.integers(0, 2 ** 15, 1000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, np.float32([3.3961776e38, 3.4e38, -3.4e38, 0.0, -0.0])])
    v = v[~np.isnan(v)]
    assert np.isnan(oracle.bf16_bits_to_f32(oracle.f32_to_bf16(np.float32([np.nan])))[0])
    ours = oracle.f32_to_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("block", [False, True])
def test_gemm_table_decode_equals_closed_form_k_loop(block):
    """The GEMM loops decode through the 256-entry table; the same sums
    written as a numpy k-ordered fp32 loop over operands decoded one element
    at a time by the closed form (or_decode), with one rounding per product
    and per add, agree bit for bit (full and sampled forms, scalar, per-row
    and block scales)."""
    rng = np.random.default_rng(31 + block)
    M, N, K = 37, 130, 384
    fa, fb = (0, 0) if block else (1, 0)
    A = _rand_codes(rng, (M, K), fa)
    B = _rand_codes(rng, (N, K), fb)
    dec = np.vectorize(lambda f, c: oracle.lib().or_decode(f, int(c)))
    Ad = dec(fa, A).astype(np.float32)
    Bd = dec(fb, B).astype(np.float32)
    if block:
        sa = (rng.random((M, K // 128)) + 0.25).astype(np.float32)
        sb = (rng.random(((N + 127) // 128, K // 128)) * 0.01 + 1e-3).astype(np.float32)
        Ah = (Ad * np.repeat(sa, 128, axis=1)).astype(np.float32)
        Bh = (Bd * np.repeat(np.repeat(sb, 128, axis=0)[:N], 128, axis=1)).astype(np.float32)
        Y, P = oracle.blockgemm(A, B, sa, sb)
    else:
        sa = (rng.random(M) + 0.5).astype(np.float32)
        sb = np.float32(0.0625)
        Ah = (Ad * sa[:, None]).astype(np.float32)
        Bh = (Bd * sb).astype(np.float32)
        Y, P = oracle.gemm(A, fa, B, fb, sa, sb)
    ref = np.zeros((M, N), np.float32)
    for k in range(K):
        ref = (ref + (Ah[:, k:k + 1] * Bh[None, :, k]).astype(np.float32)).astype(np.float32)
    assert np.array_equal(Y.view(np.uint32), ref.view(np.uint32))
    assert np.allclose(P, np.abs(Ah.astype(np.float64)) @ np.abs(Bh.astype(np.float64)).T, rtol=1e-12)
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    if block:
        y2, p2 = oracle.blockgemm_sampled(A, B, sa, sb, ms.ravel(), ns.ravel())
    else:
        y2, p2 = oracle.gemm_sampled(A, fa, B, fb, sa, sb, ms.ravel(), ns.ravel())
    assert np.array_equal(y2, Y.ravel()) and np.array_equal(p2, P.ravel())
