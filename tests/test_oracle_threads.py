"""The oracle's results do not depend on how many threads its parallel
loops use: the per-tensor quantize (amax reduction, saturation counters)
and the GEMM at one thread equal those at the default thread count."""
from __future__ import annotations

import numpy as np

import oracle


def test_oracle_results_independent_of_thread_count():
    rng = np.random.default_rng(41)
    X = (rng.standard_normal((300, 520)) * 40).astype(np.float32)
    W = rng.standard_normal((260, 520)).astype(np.float32)
    n0 = oracle.num_threads()
    outs = []
    try:
        for n in (1, max(n0, 2)):
            oracle.set_num_threads(n)
            qx = oracle.quantize(X, oracle.E4M3, "tensor")
            qw = oracle.quantize(W, oracle.E5M2, "row")
            y, p = oracle.gemm(qx["q"], oracle.E4M3, qw["q"], oracle.E5M2, qx["scale_inv"], qw["scale_inv"],
                               with_p=True)
            outs.append((qx, qw, y, p))
    finally:
        oracle.set_num_threads(n0)
    (a, b, y1, p1), (c, d, y2, p2) = outs
    for k in ("q", "scale_inv", "amax", "sat", "nonfinite", "underflow"):
        assert np.array_equal(np.asarray(a[k]), np.asarray(c[k])), k
        assert np.array_equal(np.asarray(b[k]), np.asarray(d[k])), k
    assert np.array_equal(y1, y2) and np.array_equal(p1, p2)
    assert oracle.num_threads() == n0
