"""Brute force on tiny inputs (CPU only).

For Nq, Nk <= 6 and d <= 4, every way of cutting the queries and the keys into
contiguous blocks is run through both published loop orders — the course file's
query-outer ``flash_attention_forward`` and the blog page's key-outer
Algorithm 1 (with Algorithm 2's scale and mask) — and each result must equal the
oracle's three-step definition and an independent pure-Python evaluation with
correctly rounded sums.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from oracle import tiled


def _all_cuts(n):
    inner = range(1, n)
    for r in range(n):
        yield from itertools.combinations(inner, r)


@pytest.mark.parametrize("nq,nk,d,causal", [(6, 6, 4, False), (6, 6, 4, True), (4, 6, 3, False),
                                             (6, 4, 2, True), (5, 5, 1, True), (1, 6, 4, False),
                                             (6, 1, 4, True)])
def test_every_partition_both_orders(oracle_lib, nq, nk, d, causal):
    rng = np.random.default_rng(100 * nq + 10 * nk + d + causal)
    Q, K, V = rng.standard_normal((nq, d)) * 2, rng.standard_normal((nk, d)) * 2, \
        rng.standard_normal((nk, d))
    scale = 0.7
    o_ref, l_ref = oracle.attention_f64(Q, K, V, causal, scale)

    # independent naive evaluation, row by row, exactly rounded sums
    for r in range(nq):
        o_py, l_py = tiled.naive_row_fsum(Q[r], K.tolist(), V.tolist(), r, causal, scale)
        np.testing.assert_allclose(o_ref[r], o_py, rtol=1e-14, atol=1e-15)
        assert l_ref[r] == pytest.approx(l_py, rel=1e-14, abs=1e-15)

    count = 0
    for qc in _all_cuts(nq):
        for kc in _all_cuts(nk):
            for order in (tiled.q_outer, tiled.kv_outer):
                O, L = order(Q, K, V, causal, scale, qc, kc)
                np.testing.assert_allclose(O, o_ref, rtol=1e-13, atol=1e-14)
                np.testing.assert_allclose(L, l_ref, rtol=1e-13, atol=1e-14)
                count += 1
    assert count == 2 * 2 ** (nq - 1) * 2 ** (nk - 1)


def test_course_file_demo_shape(oracle_lib):
    """The course file's exactness demo: n = 100 (not a multiple of the blocks), d = 32,
    block_q = 16, block_k = 24, fp64, causal off and on."""
    rng = np.random.default_rng(0)
    n, d = 100, 32
    Q, K, V = (rng.standard_normal((n, d)) for _ in range(3))
    scale = 1 / math.sqrt(d)
    for causal in (False, True):
        o_ref, l_ref = oracle.attention_f64(Q, K, V, causal, scale)
        O, L = tiled.q_outer(Q, K, V, causal, scale, range(16, n, 16), range(24, n, 24))
        assert np.abs(O - o_ref).max() < 1e-14 * 10
        assert np.abs(L - l_ref).max() < 1e-13
        o2, l2, _ = oracle.online_f64(Q, K, V, causal, scale, key_block=24)
        assert np.abs(o2 - o_ref).max() < 1e-14 * 10
        assert np.abs(l2 - l_ref).max() < 1e-13
