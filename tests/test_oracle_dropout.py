"""Pins of the oracle's dropout (part 4), CPU only.

Dropout acts on P after the softmax (blog page, Algorithm 2: P_dropped =
dropout(P, p), O = P_dropped V; Algorithm 4: Z regenerated from the RNG state,
dV = P_dropped^T dO, dP = dP_dropped o Z).  The pages name no generator; the reading
is Philox4x32-10 (Salmon et al., SC'11) with one 4x4 block of (query, key)
elements per call and an 8-bit threshold t.  Pins:

* the generator reproduces its published known-answer vectors
  (tests/golden/philox4x32_10_kat.json);
* t = 0 drops nothing: bitwise the oracle without dropout;
* the kept fraction and the mean of Z = keep * 256/(256 - t) match 1 - t/256 and 1
  within binomial bounds (a dropped scale or an inverted comparison fails);
* the keep decision of an element is the documented byte of the documented block;
* the dropout gradients are the derivative of the dropout forward (central finite
  differences with the mask held fixed), and sum_j dK_j = 0 still holds.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    g = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for vec in g["vectors"]:
        ctr = [int(x, 16) for x in vec["ctr"]]
        key = [int(x, 16) for x in vec["key"]]
        assert oracle.philox4x32_10(ctr, key) == [int(x, 16) for x in vec["out"]]


def test_keep_decision_is_the_documented_byte():
    seed, t, bh = 0x0123456789ABCDEF, 77, 5
    keep = oracle.dropout_keep(seed, t, bh, 9, 13)
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for q in range(9):
        for k in range(13):
            w = oracle.philox4x32_10([k >> 2, q >> 2, bh, 0], key)
            idx = 4 * (q & 3) + (k & 3)
            byte = (w[idx >> 2] >> (8 * (idx & 3))) & 0xFF
            assert keep[q, k] == (byte >= t)


@pytest.mark.parametrize("t", [1, 26, 128, 230])
def test_keep_rate_and_unbiased_scale(t):
    keep = np.concatenate([oracle.dropout_keep(1234 + s, t, s, 256, 256).ravel()
                           for s in range(4)]).astype(np.float64)
    n = keep.size
    p_keep = 1.0 - t / 256.0
    sd = math.sqrt(p_keep * (1 - p_keep) / n)
    assert abs(keep.mean() - p_keep) < 5 * sd
    z = keep * (256.0 / (256.0 - t))
    assert abs(z.mean() - 1.0) < 5 * sd * 256.0 / (256.0 - t)


def test_threshold_zero_is_no_dropout():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((20, 8)) for _ in range(3))
    dout = rng.standard_normal((20, 8))
    for causal in (False, True):
        o0, l0 = oracle.attention_f64(q, k, v, causal, 0.3)
        o1, l1 = oracle.attention_dropout_f64(q, k, v, causal, 0.3, 0, 99)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
        g0 = oracle.attention_bwd_f64(q, k, v, dout, causal, 0.3)
        g1 = oracle.attention_bwd_dropout_f64(q, k, v, dout, causal, 0.3, 0, 99)
        for a, b in zip(g0, g1):
            assert np.array_equal(a, b)


def test_dropout_changes_only_o():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((16, 8)) for _ in range(3))
    o0, l0 = oracle.attention_f64(q, k, v, False, 0.3)
    o1, l1 = oracle.attention_dropout_f64(q, k, v, False, 0.3, 64, 7)
    assert np.array_equal(l0, l1)  # L is the softmax's log-sum-exp
    assert not np.allclose(o0, o1)


@pytest.mark.parametrize("causal,t,seed", [(False, 64, 11), (True, 100, 12), (True, 200, 13)])
def test_dropout_bwd_is_the_derivative_of_the_dropout_forward(causal, t, seed):
    rng = np.random.default_rng(seed)
    nq, nk, d, bh, scale = 6, 7, 3, 2, 0.6
    q, k, v, = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    dout = rng.standard_normal((nq, d))

    def loss(q_, k_, v_):
        o, _ = oracle.attention_dropout_f64(q_, k_, v_, causal, scale, t, seed, bh)
        return float(np.sum(dout * o))

    got = oracle.attention_bwd_dropout_f64(q, k, v, dout, causal, scale, t, seed, bh)
    h = 1e-5
    for which, g in enumerate(got):
        for idx in np.ndindex(g.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            up = loss(*args)
            args[which][idx] -= 2 * h
            dn = loss(*args)
            assert abs((up - dn) / (2 * h) - g[idx]) < 1e-7 * max(1.0, abs(g[idx]))
    # each row of dS still sums to zero
    np.testing.assert_allclose(got[1].sum(axis=0), 0.0, atol=1e-12)


def test_raw_dropout_paths_agree():
    from flashattention_tiling_online_amd import inputs
    w = inputs.custom("drop_raw", 1, 2, 40, 50, 16, "bf16", True, 88)
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_do(w)
    t, seed = 51, 0xDEADBEEFCAFE
    o_r, l_r = oracle.ref_rows_dropout_f64(q, k, v, True, w.scale, "bf16", t, seed,
                                           np.repeat([0, 1], 40), np.tile(np.arange(40), 2))
    for bh in range(2):
        qw, kw, vw, dw = (oracle.widen(a, "bf16").reshape(2, -1, 16)[bh] for a in (q, k, v, dout))
        sc = np.float64(np.float32(w.scale))
        o, l = oracle.attention_dropout_f64(qw, kw, vw, True, sc, t, seed, bh)
        assert np.array_equal(o, o_r[40 * bh:40 * bh + 40])
        g = oracle.bwd_head_dropout_f64(q, k, v, dout, True, w.scale, "bf16", t, seed, bh)
        e = oracle.attention_bwd_dropout_f64(qw, kw, vw, dw, True, sc, t, seed, bh)
        for a, b in zip(g, e):
            assert np.array_equal(a, b)
