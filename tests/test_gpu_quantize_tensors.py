"""fp8_quantize_tensors on the GPU: several tensors quantized just in time
per tensor in one amax launch and one cast launch.  Each tensor's codes,
amax, scale_inv and counters must equal the oracle's per-tensor quantization
bit for bit (and so fp8_quantize's), whatever the other tensors in the call:
ragged element counts, empty tensors, an all-zero tensor, one-unit tensors,
and the 8B MLP's X and W at full size."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import FMT_NAME, dev_input, host, say

pytestmark = pytest.mark.gpu

fp8 = pytest.importorskip("fp8_precision_quantization_amd")


@pytest.fixture(autouse=True)
def _need_gpu(gpu):
    yield


def _tensor(rows, cols, in_dtype, seed, scale=2.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(rows, cols)).astype(np.float32) * scale
    return synth.to_bf16_bits(x) if in_dtype == "bf16" else x


def _check(results, xs, fmt, pow2, diags, what):
    for i, (r, x) in enumerate(zip(results, xs)):
        want = oracle.quantize(x, fmt, "tensor", pow2)
        assert np.array_equal(host(r.q), want["q"]), (what, i, x.shape, np.argwhere(host(r.q) != want["q"])[:5])
        assert host(r.amax).reshape(-1)[0] == want["amax"].reshape(-1)[0], (what, i)
        assert host(r.scale_inv).reshape(-1)[0] == want["scale_inv"].reshape(-1)[0], (what, i)
        if diags is not None and diags[i] is not None:
            d = diags[i].read()
            assert (d["sat"], d["nonfinite"], d["underflow"]) == (want["sat"], want["nonfinite"],
                                                                   want["underflow"]), (what, i)


SMALL = [(300, 515), (1, 1), (0, 5), (3, 3), (1024, 1000), (257, 129), (8, 1), (64, 64)]


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pow2", [False, True])
def test_quantize_tensors_parity(fmt, in_dtype, pow2):
    """Eight tensors of different sizes and ranges (one all zero, one empty,
    ragged counts), each against the oracle; every second one counts."""
    xs = [_tensor(r, c, in_dtype, 500 + i, scale=2.0 ** (3 * i - 9)) for i, (r, c) in enumerate(SMALL)]
    xs[7] = np.zeros_like(xs[7])
    diags = [fp8.Diag() if i % 2 == 0 else None for i in range(len(xs))]
    say("quantize_tensors", FMT_NAME[fmt], in_dtype, "pow2" if pow2 else "", [x.shape for x in xs])
    rs = fp8.quantize_tensors([dev_input(x) for x in xs], FMT_NAME[fmt], pow2=pow2, diags=diags)
    _check(rs, xs, fmt, pow2, diags, "small")
    assert host(rs[7].scale_inv).reshape(-1)[0] == 1.0 and host(rs[2].scale_inv).reshape(-1)[0] == 1.0


@pytest.mark.parametrize("n", [1, 2, 5])
def test_quantize_tensors_equals_single_calls(n):
    """Codes and scales of every tensor equal the single-tensor call's."""
    shapes = [(513, 777), (2048, 1031), (5, 4096), (999, 8), (4096, 17)][:n]
    xs = [_tensor(r, c, "bf16", 40 + i) for i, (r, c) in enumerate(shapes)]
    dx = [dev_input(x) for x in xs]
    say("quantize_tensors vs single calls", n)
    rs = fp8.quantize_tensors(dx, "e4m3")
    for i, x in enumerate(dx):
        one = fp8.quantize(x, "e4m3", "tensor")
        assert np.array_equal(host(rs[i].q), host(one.q)), i
        assert host(rs[i].scale_inv)[0, 0] == host(one.scale_inv).reshape(-1)[0], i
        assert host(rs[i].amax)[0, 0] == host(one.amax).reshape(-1)[0], i


@pytest.mark.timeout(600)
def test_quantize_tensors_mlp8b_sizes_repeated():
    """X [4096 x 4096] and W [14336 x 4096] bf16 (Student-t(4) and
    N(0, 0.015), the 8B MLP workload's operands) in one call, twice in a
    row on one stream, then with a small third tensor added: bit-exact with
    the oracle, counters included."""
    X, W = synth.mlp8b()
    wx, ww = oracle.quantize(X, oracle.E4M3, "tensor"), oracle.quantize(W, oracle.E4M3, "tensor")
    dX, dW = dev_input(X), dev_input(W)
    for rep in range(2):
        say("quantize_tensors mlp8b X, W", rep)
        diags = [fp8.Diag(), fp8.Diag()]
        rs = fp8.quantize_tensors([dX, dW], "e4m3", diags=diags)
        for r, want, d in zip(rs, (wx, ww), diags):
            assert np.array_equal(host(r.q), want["q"]), rep
            assert host(r.amax)[0, 0] == want["amax"].reshape(-1)[0]
            assert host(r.scale_inv)[0, 0] == want["scale_inv"].reshape(-1)[0]
            c = d.read()
            assert (c["sat"], c["nonfinite"], c["underflow"]) == (want["sat"], want["nonfinite"], want["underflow"])
    small = _tensor(33, 65, "bf16", 7)
    say("quantize_tensors mlp8b X, small, W")
    rs = fp8.quantize_tensors([dX, dev_input(small), dW], "e4m3")
    _check([rs[1]], [small], oracle.E4M3, False, None, "small between")
    assert np.array_equal(host(rs[0].q), wx["q"]) and np.array_equal(host(rs[2].q), ww["q"])
