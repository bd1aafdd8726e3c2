"""GPU parity of amax / scale / cast against the CPU oracle: codes, amax and
scale_inv bit-exact; diagnostic counters exact.  Shapes span several tiles
and ragged tails (columns not a multiple of 8 or 128, rows not a multiple of
4 or 128), strided inputs and outputs, and the degenerate cases."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import (FMAX, FMT_NAME, crafted_history, dev_input, dev_u8, host, say)

pytestmark = pytest.mark.gpu

fp8 = pytest.importorskip("fp8_precision_quantization_amd")

FMTS = [oracle.E4M3, oracle.E5M2]


@pytest.fixture(autouse=True)
def _need_gpu(gpu):
    yield


# ------------------------------------------------------------------ codec --
def _quantize_fixed_scale(x: np.ndarray, fmt, scale_pow2_k: int = 0, diag=None):
    """Delayed call on a crafted history: s = 2^k exactly."""
    hist = fp8.AmaxHistory(16)
    hist.buf.copy_(crafted_history(FMAX[fmt] / 2.0 ** scale_pow2_k))
    xt = dev_input(x)
    r = fp8.quantize(xt, FMT_NAME[fmt], "tensor", history=hist, diag=diag)
    return r, hist


@pytest.mark.parametrize("fmt", FMTS)
def test_codec_all_bf16_patterns(fmt):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    f = synth.bf16_bits_to_f32(bits)
    bits = np.where(np.isnan(f), np.uint16(0), bits)          # NaN has its own test
    say("codec bf16 all patterns", FMT_NAME[fmt])
    diag = fp8.Diag()
    r, _ = _quantize_fixed_scale(bits, fmt, 0, diag)
    got = host(r.q)
    want, cnt = oracle.quantize_with_scales(bits, fmt, "tensor", np.float32([1.0]))
    assert host(r.scale_inv)[0] == 1.0
    mism = np.argwhere(got != want)
    assert mism.size == 0, (mism[:8].tolist(), got[tuple(mism[0])], want[tuple(mism[0])])
    d = diag.read()
    assert d["sat"] == cnt["sat"] and d["nonfinite"] == cnt["nonfinite"] and d["underflow"] == cnt["underflow"]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("k", [0, 3, -5])
def test_codec_fp32_random_and_midpoints(fmt, k):
    rng = np.random.default_rng(100 + k)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    t = oracle.decode_table(fmt)
    pos = t[:128][np.isfinite(t[:128])]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32) / np.float32(2.0 ** k)
    extra = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
                            pos.astype(np.float32) / np.float32(2.0 ** k),
                            np.float32([np.inf, -np.inf, 0.0, -0.0, 1e-45, -1e-45, 3.4e38])])
    v = np.concatenate([v, extra, -extra])
    v = np.where(np.isnan(v), np.float32(0), v)
    pad = (-v.size) % 1024
    v = np.concatenate([v, np.zeros(pad, np.float32)]).reshape(-1, 1024)
    say("codec fp32 random", FMT_NAME[fmt], "k", k)
    r, _ = _quantize_fixed_scale(v, fmt, k)
    got = host(r.q)
    want, _ = oracle.quantize_with_scales(v, fmt, "tensor", np.float32([2.0 ** k]))
    assert host(r.scale_inv)[0] == np.float32(2.0 ** -k)
    mism = np.argwhere(got != want)
    assert mism.size == 0, (mism[:8].tolist(), v[tuple(mism[0])], got[tuple(mism[0])], want[tuple(mism[0])])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", FMTS)
def test_codec_exhaustive_over_active_binades(fmt):
    """Every fp32 of both signs in the binades where an FP8 code varies
    (from two binades below the smallest subnormal to the one past the
    largest value: E4M3 21, E5M2 35 binades of 2^23 values) through the
    GPU cast at scale 1.0, against the oracle, one binade per call."""
    from tests.test_oracle_pins import active_binades, binade_bits
    for e in active_binades(fmt):
        for sg in (0, 1):
            v = binade_bits(e, sg).view(np.float32).reshape(-1, 4096)
            say("codec binade", FMT_NAME[fmt], e, sg)
            r, _ = _quantize_fixed_scale(v, fmt, 0)
            got = host(r.q)
            want, _ = oracle.quantize_with_scales(v, fmt, "tensor", np.float32([1.0]))
            mism = np.argwhere(got != want)
            assert mism.size == 0, (e, sg, mism[:4].tolist(), v[tuple(mism[0])], got[tuple(mism[0])],
                                    want[tuple(mism[0])])


@pytest.mark.parametrize("fmt", FMTS)
def test_codec_nan_inputs(fmt):
    payloads = np.array([0x7FC00000, 0x7F800001, 0x7FFFFFFF, 0xFFC00000, 0xFF800001, 0xFFFFFFFF],
                        np.uint32).view(np.float32)
    x = np.zeros((1, 64), np.float32)
    x[0, :6] = payloads
    x[0, 6:10] = [1.0, -2.0, 3.5, -0.0]
    say("codec NaN", FMT_NAME[fmt])
    r, _ = _quantize_fixed_scale(x, fmt, 0)
    got = host(r.q)
    want, _ = oracle.quantize_with_scales(x, fmt, "tensor", np.float32([1.0]))
    assert np.array_equal(got, want), (got[0, :10], want[0, :10])


# ------------------------------------------------------------- quantize --
SHAPES = [(1, 1), (3, 7), (4, 8), (129, 130), (260, 515), (512, 1024), (33, 4100)]


def _inputs(rows, cols, in_dtype, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(rows, cols)).astype(np.float32) * 2
    if rows > 2:
        x[1, :] = 0.0                                # an all-zero row
    if cols > 5:
        x[:, 5] *= 300                               # an outlier column
    return synth.to_bf16_bits(x) if in_dtype == "bf16" else x


@pytest.mark.parametrize("gran", ["tensor", "row", "1x128", "128x128"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pow2", [False, True])
def test_quantize_parity(gran, fmt, in_dtype, pow2):
    for i, (rows, cols) in enumerate(SHAPES):
        x = _inputs(rows, cols, in_dtype, 1000 + i)
        say("quantize", gran, FMT_NAME[fmt], in_dtype, "pow2" if pow2 else "", rows, cols)
        diag = fp8.Diag()
        r = fp8.quantize(dev_input(x), FMT_NAME[fmt], gran, pow2=pow2, diag=diag)
        want = oracle.quantize(x, fmt, gran, pow2)
        got_q = host(r.q)
        assert np.array_equal(got_q, want["q"]), (rows, cols, np.argwhere(got_q != want["q"])[:5])
        assert np.array_equal(host(r.amax).reshape(-1), want["amax"].reshape(-1))
        assert np.array_equal(host(r.scale_inv).reshape(-1), want["scale_inv"].reshape(-1))
        d = diag.read()
        assert (d["sat"], d["nonfinite"], d["underflow"]) == (want["sat"], want["nonfinite"], want["underflow"])


@pytest.mark.parametrize("gran", ["tensor", "row", "1x128", "128x128"])
def test_quantize_strided_in_and_out(gran):
    rows, cols = 200, 300
    x = _inputs(rows, 320, "bf16", 7)            # ld = 320 > cols
    xt = dev_input(x)[:, :cols]
    out = torch.full((rows, 336), 0xAB, dtype=torch.uint8, device="cuda")[:, :cols]
    say("quantize strided", gran)
    r = fp8.quantize(xt, "e4m3", gran, out=out)
    want = oracle.quantize(np.ascontiguousarray(x[:, :cols]), oracle.E4M3, gran)
    assert np.array_equal(host(r.q), want["q"])
    full = host(out.as_strided((rows, 336), (336, 1)))
    assert np.all(full[:, cols:] == 0xAB)        # padding untouched


@pytest.mark.parametrize("gran", ["tensor", "row", "1x128", "128x128"])
@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_amax_api(gran, in_dtype):
    for i, (rows, cols) in enumerate(SHAPES):
        x = _inputs(rows, cols, in_dtype, 2000 + i)
        say("amax", gran, in_dtype, rows, cols)
        got = host(fp8.amax(dev_input(x), gran))
        assert np.array_equal(got.reshape(-1), oracle.amax(x, gran).reshape(-1))


def test_amax_nonfinite():
    x = np.ones((130, 260), np.float32)
    x[3, 4] = np.inf
    x[129, 259] = np.nan
    for gran in ["tensor", "row", "1x128", "128x128"]:
        say("amax nonfinite", gran)
        got = host(fp8.amax(dev_input(x), gran)).reshape(-1)
        want = oracle.amax(x, gran).reshape(-1)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_quantize_row_two_pass_long_rows():
    x = _inputs(5, 9000, "bf16", 3)                 # more than 4096 elements per row
    say("quantize long rows")
    r = fp8.quantize(dev_input(x), "e4m3", "row", pow2=True)
    want = oracle.quantize(x, oracle.E4M3, "row", True)
    assert np.array_equal(host(r.q), want["q"])
    assert np.array_equal(host(r.scale_inv).reshape(-1), want["scale_inv"].reshape(-1))


@pytest.mark.parametrize("shape", [(0, 5), (5, 0), (0, 0)])
@pytest.mark.parametrize("gran", ["tensor", "row"])
def test_quantize_empty(shape, gran):
    x = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    say("quantize empty", shape, gran)
    r = fp8.quantize(x, "e4m3", gran)
    want = oracle.quantize(np.zeros(shape, np.uint16), oracle.E4M3, gran)
    assert np.array_equal(host(r.amax).reshape(-1), want["amax"].reshape(-1))
    assert np.array_equal(host(r.scale_inv).reshape(-1), want["scale_inv"].reshape(-1))


def test_quantize_all_zero_and_subnormal_inputs():
    x = np.zeros((64, 64), np.float32)
    say("quantize all zero")
    r = fp8.quantize(dev_input(x), "e4m3", "tensor")
    assert host(r.scale_inv)[0] == 1.0 and np.all(host(r.q) == 0)
    # a tensor of binary32 subnormals: the scale overflows to FLT_MAX
    x = np.full((16, 64), 1e-39, np.float32)
    x[3, 3] = -2e-39
    say("quantize subnormal")
    r = fp8.quantize(dev_input(x), "e4m3", "tensor")
    want = oracle.quantize(x, oracle.E4M3, "tensor")
    assert np.array_equal(host(r.q), want["q"])
    assert np.array_equal(host(r.scale_inv), want["scale_inv"].reshape(-1))


# ------------------------------------------------------------ transposed --
@pytest.mark.parametrize("shape", [(300, 515), (128, 128), (1, 1), (257, 129), (1024, 640)])
@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_transposed(shape, fmt):
    rows, cols = shape
    x = _inputs(rows, cols, "bf16", 77)
    say("quantize transposed", shape, FMT_NAME[fmt])
    diag = fp8.Diag()
    r = fp8.quantize(dev_input(x), FMT_NAME[fmt], "tensor", transpose=True, diag=diag)
    want = oracle.quantize(x, fmt, "tensor")
    got = host(r.q)
    assert got.shape == (cols, rows)
    assert np.array_equal(got, want["q"].T)
    assert host(r.scale_inv)[0] == want["scale_inv"][0, 0]
    d = diag.read()
    assert (d["sat"], d["underflow"]) == (want["sat"], want["underflow"])


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_transposed_and_dual_many_tiles(fmt):
    """More 128x128 tiles (33 x 40 = 1320) than the transposed cast's grid
    (4 blocks per CU), so blocks walk several tiles, ragged ones included,
    with the next tile's loads in flight: the transposed codes, and both
    layouts of the dual cast, against the oracle."""
    rows, cols = 4100, 5000
    x = _inputs(rows, cols, "bf16", 78)
    want = oracle.quantize(x, fmt, "tensor")
    xt = dev_input(x)
    say("quantize transposed many tiles", FMT_NAME[fmt])
    r = fp8.quantize(xt, FMT_NAME[fmt], "tensor", transpose=True)
    assert np.array_equal(host(r.q), want["q"].T)
    assert host(r.scale_inv)[0] == want["scale_inv"][0, 0]
    say("quantize dual many tiles", FMT_NAME[fmt])
    rd, qt = fp8.quantize_dual(xt, FMT_NAME[fmt])
    assert np.array_equal(host(rd.q), want["q"]) and np.array_equal(host(qt), want["q"].T)
    assert host(rd.scale_inv)[0] == want["scale_inv"][0, 0]


@pytest.mark.parametrize("shape", [(7000, 3000), (5000, 4104)])
def test_quantize_rows_persistent_loop(shape):
    """More rows than the row cast's persistent grid has waves (3 blocks of 4
    waves per CU), so every wave loops over rows with the next row's loads in
    flight: ragged rows held in registers (3000) and rows past 4096 elements
    (the two-read path); codes, per-row scales and amaxes, counters."""
    rows, cols = shape
    x = _inputs(rows, cols, "bf16", 79)
    say("quantize rows persistent", shape)
    diag = fp8.Diag()
    r = fp8.quantize(dev_input(x), "e4m3", "row", pow2=True, diag=diag)
    want = oracle.quantize(x, oracle.E4M3, "row", True)
    assert np.array_equal(host(r.q), want["q"])
    assert np.array_equal(host(r.scale_inv).reshape(-1), want["scale_inv"].reshape(-1))
    assert np.array_equal(host(r.amax).reshape(-1), want["amax"].reshape(-1))
    d = diag.read()
    assert (d["sat"], d["nonfinite"], d["underflow"]) == (want["sat"], want["nonfinite"], want["underflow"])


# ---------------------------------------------------------------- delayed --
@pytest.mark.parametrize("transpose", [False, True])
def test_delayed_ring_20_steps(transpose):
    """The wgrad recipe at a reduced size, step by step against the oracle
    ring: codes, scale_inv, amax, saturation counts and the ring itself."""
    tokens, hidden = 512, 384
    h_dy, h_x = fp8.AmaxHistory(16), fp8.AmaxHistory(16)
    o_dy, o_x = oracle.DelayedScaler(oracle.E5M2), oracle.DelayedScaler(oracle.E4M3)
    for t in range(20):
        dy, x = synth.wgrad_step(t, tokens=tokens, hidden=hidden)
        for name, data, h, o, fmt in (("dY", dy, h_dy, o_dy, "e5m2"), ("X", x, h_x, o_x, "e4m3")):
            say("delayed step", t, name, "transpose" if transpose else "")
            diag = fp8.Diag()
            r = fp8.quantize(dev_input(data), fmt, "tensor", history=h, transpose=transpose, diag=diag)
            w = o.step(data)
            got = host(r.q)
            assert np.array_equal(got, w["q"].T if transpose else w["q"]), (t, name)
            assert host(r.scale_inv)[0] == w["scale_inv"], (t, name)
            assert host(r.amax)[0] == w["amax"], (t, name)
            assert diag.read()["sat"] == w["sat"], (t, name)
            st, os_ = h.state(), o.state()
            assert (st["count"], st["pos"]) == (os_["count"], os_["pos"])
            assert np.array_equal(st["amax"].numpy(), os_["amax"])
            if st["count"] > 0:
                s_next, _ = oracle.scale(o.window_max(), fmt)
                assert st["scale"] == s_next
        if t == 12:
            assert o_dy.state()["count"] == 13


@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("with_diag", [False, True])
def test_delayed_spike_guard_20_steps(transpose, with_diag):
    """The spike guard with threshold 10 on the wgrad recipe, step by step
    against the oracle: only dY's spike step casts again just in time (codes,
    scale_inv, saturation count of that cast), everything else and the rings
    as without the guard; the history counts one re-cast."""
    tokens, hidden = 512, 384
    h_dy, h_x = fp8.AmaxHistory(16), fp8.AmaxHistory(16)
    h_dy.set_guard(10.0)
    h_x.set_guard(10.0)
    o_dy = oracle.DelayedScaler(oracle.E5M2, spike_threshold=10.0)
    o_x = oracle.DelayedScaler(oracle.E4M3, spike_threshold=10.0)
    for t in range(20):
        dy, x = synth.wgrad_step(t, tokens=tokens, hidden=hidden)
        for name, data, h, o, fmt in (("dY", dy, h_dy, o_dy, "e5m2"), ("X", x, h_x, o_x, "e4m3")):
            say("guarded step", t, name, "transpose" if transpose else "", "diag" if with_diag else "")
            diag = fp8.Diag() if with_diag else None
            r = fp8.quantize(dev_input(data), fmt, "tensor", history=h, transpose=transpose, diag=diag,
                             spike_guard=True)
            w = o.step(data)
            assert w["spiked"] == (name == "dY" and t == 12)
            got = host(r.q)
            assert np.array_equal(got, w["q"].T if transpose else w["q"]), (t, name)
            assert host(r.scale_inv)[0] == w["scale_inv"], (t, name)
            assert host(r.amax)[0] == w["amax"], (t, name)
            if with_diag:
                assert diag.read()["sat"] == w["sat"], (t, name)
            st, os_ = h.state(), o.state()
            assert (st["count"], st["pos"]) == (os_["count"], os_["pos"])
            assert np.array_equal(st["amax"].numpy(), os_["amax"])
            assert st["last_spiked"] == int(w["spiked"])
    assert h_dy.state()["spikes"] == 1 and h_x.state()["spikes"] == 0
    assert h_dy.state()["spike_threshold"] == 10.0


@pytest.mark.parametrize("case", ["flat_bf16", "strided_bf16", "flat_f32", "transposed_f32", "dual_bf16"])
def test_delayed_bootstrap_in_cast_many_workgroups(case):
    """Delayed casts on a tensor that takes about a thousand workgroups:
    step 0 (an empty history: inside the cast, one workgroup reads the whole
    tensor for the just-in-time bootstrap while the others wait for it) and
    four more steps against the oracle ring; the history's sync words are
    zero after every call; a reset history bootstraps again."""
    rows, cols = 3000, 4104
    rng = np.random.default_rng(77)
    f32 = case.endswith("f32")
    h = fp8.AmaxHistory(16)
    o = oracle.DelayedScaler(oracle.E5M2)
    for t in range(7):
        if t == 5:                   # start over from an empty history
            h.reset()
            o = oracle.DelayedScaler(oracle.E5M2)
        x = (rng.standard_t(3, size=(rows, cols)) * 1e-3 * (1.0 + t)).astype(np.float32)
        data = x if f32 else synth.to_bf16_bits(x)
        say("delayed bootstrap in cast", case, "step", t)
        if case == "strided_bf16":
            wide = np.zeros((rows, cols + 40), dtype=np.uint16)
            wide[:, :cols] = data
            xt = dev_input(wide)[:, :cols]
        else:
            xt = dev_input(data)
        diag = fp8.Diag()
        if case == "dual_bf16":
            r, qt = fp8.quantize_dual(xt, "e5m2", history=h, diag=diag)
        else:
            r = fp8.quantize(xt, "e5m2", "tensor", history=h, transpose=case.startswith("transposed"), diag=diag)
        w = o.step(data)
        got = host(r.q)
        assert np.array_equal(got, w["q"].T if case.startswith("transposed") else w["q"]), (case, t)
        if case == "dual_bf16":
            assert np.array_equal(host(qt), w["q"].T), (case, t)
        assert host(r.scale_inv)[0] == w["scale_inv"] and host(r.amax)[0] == w["amax"], (case, t)
        assert diag.read()["sat"] == w["sat"], (case, t)
        st, os_ = h.state(), o.state()
        assert (st["count"], st["pos"]) == (os_["count"], os_["pos"]), (case, t)
        assert np.array_equal(st["amax"].numpy(), os_["amax"]), (case, t)
        assert st["steps"] == (t + 1 if t < 5 else t - 4), (case, t)
        words = host(h.buf)
        assert np.all(words[26:32] == 0), (case, t, words[26:32])


def test_delayed_save_restore():
    tokens, hidden = 256, 256
    h = fp8.AmaxHistory(16)
    ref = []
    for t in range(14):
        dy, _ = synth.wgrad_step(t, tokens=tokens, hidden=hidden)
        say("delayed uninterrupted", t)
        r = fp8.quantize(dev_input(dy), "e5m2", "tensor", history=h)
        ref.append((host(r.q), host(r.scale_inv)[0]))
        if t == 9:
            saved = h.save()
    h2 = fp8.AmaxHistory(16)
    h2.load(saved)
    for t in range(10, 14):
        dy, _ = synth.wgrad_step(t, tokens=tokens, hidden=hidden)
        say("delayed restored", t)
        r = fp8.quantize(dev_input(dy), "e5m2", "tensor", history=h2)
        assert np.array_equal(host(r.q), ref[t][0]) and host(r.scale_inv)[0] == ref[t][1]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("with_diag", [False, True])
def test_quantize_tensor_large_sizes_repeated(with_diag):
    """Per-tensor just-in-time casts at the workloads' sizes and beyond
    (ragged columns, fp32 inputs, 128 Mi elements), each twice in a row on
    one stream so the second call reuses the scratch the first left: codes,
    amax, scale and the saturation counters bit-exact with the oracle."""
    for rows, cols, in_dtype in [(4096, 4096, "bf16"), (4096, 4104, "bf16"), (14336, 4096, "bf16"),
                                 (16384, 8192, "bf16"), (2048, 4096, "f32"), (6000, 4096, "f32")]:
        x = _inputs(rows, cols, in_dtype, rows + cols)
        want = oracle.quantize(x, oracle.E4M3, "tensor")
        xt = dev_input(x)
        for rep in range(2):
            say("quantize tensor size", rows, cols, in_dtype, "diag" if with_diag else "", rep)
            diag = fp8.Diag() if with_diag else None
            r = fp8.quantize(xt, "e4m3", "tensor", diag=diag)
            assert np.array_equal(host(r.q), want["q"]), (rows, cols, rep)
            assert host(r.amax).reshape(-1)[0] == want["amax"].reshape(-1)[0]
            assert host(r.scale_inv).reshape(-1)[0] == want["scale_inv"].reshape(-1)[0]
            if with_diag:
                d = diag.read()
                assert (d["sat"], d["nonfinite"], d["underflow"]) == (want["sat"], want["nonfinite"],
                                                                       want["underflow"])
        del xt


def test_quantize_deterministic_and_stream_ordered():
    x = _inputs(1000, 2000, "bf16", 9)
    xt = dev_input(x)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        say("quantize on side stream")
        a = fp8.quantize(xt, "e4m3", "tensor")
        b = fp8.quantize(xt, "e4m3", "tensor")
    s.synchronize()
    assert torch.equal(a.q, b.q) and torch.equal(a.scale_inv, b.scale_inv)


def test_invalid_args_on_gpu_raise():
    x = torch.zeros((4, 4), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fp8.Fp8Error) as e:
        fp8.quantize(x, "e4m3", "row", transpose=True)
    assert "TRANSPOSE" in str(e.value)
    with pytest.raises(fp8.Fp8Error):
        fp8.quantize(x, 7, "tensor")


def test_binding_rejects_wrong_buffers():
    """Output and scale buffers of the wrong dtype, size, layout or device
    raise in the binding before any launch (the library itself only sees
    pointers)."""
    dev = "cuda"
    x = torch.zeros((64, 256), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="out must have shape"):
        fp8.quantize(x, "e4m3", "tensor", out=torch.empty((64, 255), dtype=torch.uint8, device=dev))
    with pytest.raises(TypeError, match="out must be"):
        fp8.quantize(x, "e4m3", "tensor", out=torch.empty((64, 256), dtype=torch.int8, device=dev))
    with pytest.raises(ValueError, match="out must have shape"):
        fp8.quantize(x, "e4m3", "tensor", transpose=True, out=torch.empty((64, 256), dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="scale_inv_out must be a contiguous tensor of 64"):
        fp8.quantize(x, "e4m3", "row", scale_inv_out=torch.empty(63, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError, match="amax_out must be a contiguous tensor of 128"):
        fp8.quantize(x, "e4m3", "1x128", amax_out=torch.empty((64, 4), dtype=torch.float32, device=dev)[:, ::2])
    with pytest.raises(ValueError, match="scale_inv_out must be a tensor on"):
        fp8.quantize(x, "e4m3", "tensor", scale_inv_out=torch.empty(1, dtype=torch.float32))
    with pytest.raises(ValueError, match="out_t must have shape"):
        fp8.quantize_dual(x, out_t=torch.empty((64, 256), dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="out must be a contiguous tensor of 128"):
        fp8.amax(x, "1x128", out=torch.empty(3, dtype=torch.float32, device=dev))
    a = torch.zeros((64, 256), dtype=torch.uint8, device=dev)
    b = torch.zeros((128, 256), dtype=torch.uint8, device=dev)
    one = torch.ones(1, dtype=torch.float32, device=dev)
    with pytest.raises(TypeError, match="a_scale_inv must be"):
        fp8.scaled_gemm(a, b, one.double(), one)
    with pytest.raises(ValueError, match="out must have shape"):
        fp8.scaled_gemm(a, b, one, one, out=torch.empty((64, 127), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError, match="b_q must be"):
        fp8.scaled_gemm(a, b.cpu(), one, one)
    with pytest.raises(ValueError, match="a_scale_inv must be a contiguous tensor of 128"):
        fp8.blockscaled_gemm(a, b, torch.ones(64, dtype=torch.float32, device=dev),
                             torch.ones(2, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError, match="b_scale_inv must be a contiguous tensor of 2"):
        fp8.blockscaled_gemm(a, b, torch.ones((64, 2), dtype=torch.float32, device=dev),
                             torch.ones(1, dtype=torch.float32, device=dev))
    offs = torch.tensor([0, 32, 64], dtype=torch.int32, device=dev)
    bg = torch.zeros((2, 128, 256), dtype=torch.uint8, device=dev)
    with pytest.raises(TypeError, match="b_scale_inv must be"):
        fp8.grouped_gemm(a, bg, offs, one, torch.ones(2, dtype=torch.float16, device=dev))
    cache = fp8.KVTensorCache(16, 2, 128)
    with pytest.raises(ValueError, match="scale_inv must be a contiguous tensor of 32"):
        fp8.kv_store(torch.zeros((4, 256), dtype=torch.bfloat16, device=dev), cache.data,
                     torch.zeros(31, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError, match="scale_inv must be a contiguous tensor of 32"):
        fp8.kv_load(cache.data, torch.zeros((16, 2), dtype=torch.float32, device=dev).t(), n=4)
    torch.cuda.synchronize()
