"""Pins of the oracle's grouped scaled GEMM (grouped_gemm_sampled,
group_of_rows) against a brute-force row scan, numpy fp64 products of the
decoded operands, the reduction to the plain GEMM with one group, and exact
integer sums.

Page: "DeepL bets on FP8" (hmyw.cn), section 3.2 (MoE: tokens grouped by
route, each group multiplied with its own expert's weight)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests.gpu_util import random_codes


def _brute_group(offsets, m):
    for g in range(len(offsets) - 1):
        if offsets[g] <= m < offsets[g + 1]:
            return g
    return -1


def test_group_of_rows_brute_force():
    rng = np.random.default_rng(1)
    for _ in range(50):
        G = int(rng.integers(1, 9))
        sizes = rng.integers(0, 6, G)
        start = int(rng.integers(0, 3))
        offsets = np.concatenate([[start], start + np.cumsum(sizes)])
        ms = np.arange(offsets[-1] + 3)
        got = oracle.group_of_rows(offsets, ms)
        ref = np.array([_brute_group(offsets, m) for m in ms])
        assert np.array_equal(got, ref), (offsets, got, ref)


def _problem(G, N, K, sizes, seed, fa=oracle.E4M3, fb=oracle.E4M3):
    rng = np.random.default_rng(seed)
    M = int(np.sum(sizes)) + 5                       # 5 trailing rows in no group
    A = random_codes(rng, (M, K), fa)
    B = random_codes(rng, (G, N, K), fb)
    a_inv = (2.0 ** rng.uniform(-6, 2, M)).astype(np.float32)
    b_inv = (2.0 ** rng.uniform(-6, 2, (G, N))).astype(np.float32)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    return A, B, a_inv, b_inv, offsets


def test_grouped_one_group_is_the_plain_gemm():
    A, B, a_inv, b_inv, offsets = _problem(1, 40, 96, [30], 2)
    ms = np.repeat(np.arange(30), 40)
    ns = np.tile(np.arange(40), 30)
    y, p = oracle.grouped_gemm_sampled(A, 0, B, 0, offsets, a_inv, b_inv, ms, ns)
    y1, p1 = oracle.gemm_sampled(A, 0, B[0], 0, a_inv, b_inv[0], ms, ns)
    assert np.array_equal(y, y1) and np.array_equal(p, p1)


@pytest.mark.parametrize("per_row_b", [False, True])
@pytest.mark.parametrize("fmts", [(oracle.E4M3, oracle.E4M3), (oracle.E5M2, oracle.E4M3)])
def test_grouped_vs_numpy_per_group_products(per_row_b, fmts):
    """Every output against the fp64 product of the decoded, scaled operands
    of its own expert: within the fp32 accumulation bound K * 2^-24 * P; the
    rows in no group are NaN; P equals the fp64 sum of |products|."""
    fa, fb = fmts
    G, N, K = 4, 24, 80
    sizes = [7, 0, 13, 3]
    A, B, a_inv, b_inv, offsets = _problem(G, N, K, sizes, 3, fa, fb)
    if not per_row_b:
        b_inv = b_inv[:, :1].copy()
    M = A.shape[0]
    ms = np.repeat(np.arange(M), N)
    ns = np.tile(np.arange(N), M)
    y, p = oracle.grouped_gemm_sampled(A, fa, B, fb, offsets, a_inv, b_inv, ms, ns)
    ta, tb = oracle.decode_table(fa), oracle.decode_table(fb)
    Ad = (ta[A] * a_inv[:, None].astype(np.float32)).astype(np.float32).astype(np.float64)
    y = y.reshape(M, N)
    p = p.reshape(M, N)
    for g in range(G):
        rows = slice(offsets[g], offsets[g + 1])
        sb = b_inv[g][:, None] if per_row_b else b_inv[g, 0]
        Bd = (tb[B[g]] * np.float32(1) * sb).astype(np.float32).astype(np.float64)
        ref = Ad[rows] @ Bd.T
        pref = np.abs(Ad[rows]) @ np.abs(Bd).T
        assert np.allclose(p[rows], pref, rtol=1e-12, atol=0)
        assert (np.abs(y[rows] - ref) <= K * 2.0 ** -24 * pref + 1e-300).all()
    assert np.isnan(y[offsets[-1]:]).all()


def test_grouped_wrong_expert_is_detected():
    """A row routed to its neighbour's expert changes its outputs: the
    routing is not a no-op the pins above could miss."""
    G, N, K = 3, 16, 64
    A, B, a_inv, b_inv, offsets = _problem(G, N, K, [5, 5, 5], 4)
    ms = np.repeat(np.arange(15), N)
    ns = np.tile(np.arange(N), 15)
    y, _ = oracle.grouped_gemm_sampled(A, 0, B, 0, offsets, a_inv, b_inv, ms, ns)
    shifted = offsets.copy()
    shifted[1] += 1                       # row 5 moves from expert 1 to expert 0
    y2, _ = oracle.grouped_gemm_sampled(A, 0, B, 0, shifted, a_inv, b_inv, ms, ns)
    diff = np.nonzero(y.reshape(15, N) != y2.reshape(15, N))[0]
    assert set(diff.tolist()) == {5}


def test_grouped_exact_matches_integer_sums():
    """The exact form: every output equals the integer dot product of the
    codes' integer significands, scaled exactly (computed here with Python
    integers and fractions for a few outputs)."""
    from fractions import Fraction
    G, N, K = 2, 8, 32
    A, B, a_inv, b_inv, offsets = _problem(G, N, K, [3, 4], 5)
    ms = np.array([0, 2, 3, 6, 6])
    ns = np.array([0, 7, 3, 1, 5])
    ye = oracle.grouped_gemm_sampled(A, 0, B, 0, offsets, a_inv, b_inv, ms, ns, exact=True)
    t = oracle.decode_table(0)
    for i, (m, n) in enumerate(zip(ms, ns)):
        g = _brute_group(offsets, m)
        s = sum(Fraction(float(t[A[m, k]])) * Fraction(float(t[B[g, n, k]])) for k in range(K))
        ref = s * Fraction(float(a_inv[m])) * Fraction(float(b_inv[g, n]))
        assert ye[i] == float(ref)
