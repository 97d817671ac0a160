"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage it pins.  Together they are chosen so that a dropped
term, a wrong sign or index, or a transposed operand anywhere in the oracle
fails at least one of them (the mutation tests at the end plant such mistakes
in a copy of the oracle and check that the pins catch them).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import tiled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# P1 — the worked example ("手写 Flash Attention", section 2.2)
# ---------------------------------------------------------------------------

def test_worked_example_intermediates_and_final(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    x, block, pr = g["scores"], g["block"], g["printed"]
    tol = 0.5 * 10 ** -g["printed_decimals"] + 1e-12  # printed to 3 decimals
    y, tr = oracle.softmax_online(x, block)

    assert tr["run_m"][0] == pr["block1_max"]
    assert tr["run_l"][0] == pytest.approx(pr["block1_sum"], abs=tol)
    # the block-1 exponentials and local softmax follow from m_1 and l_1
    e1 = [math.exp(v - tr["run_m"][0]) for v in x[:2]]
    assert e1 == pytest.approx(pr["block1_exp"], abs=tol)
    assert [v / tr["run_l"][0] for v in e1] == pytest.approx(pr["block1_local_softmax"], abs=tol)
    assert tr["run_m"][1] == pr["block2_max"]
    assert tr["carried"][1] == pytest.approx(pr["block1_sum_rebased"], abs=tol)
    assert tr["fresh"][1] == pytest.approx(pr["block2_sum"], abs=tol)
    assert tr["run_l"][1] == pytest.approx(pr["total_sum"], abs=tol)
    assert y[2] == pytest.approx(pr["final_softmax"][2], abs=tol)

    # closed form of the final vector and of the logsumexp
    z = math.fsum(math.exp(v - 5.0) for v in x)
    assert y == pytest.approx([math.exp(v - 5.0) / z for v in x], rel=1e-15, abs=0)
    assert tr["run_m"][1] + math.log(tr["run_l"][1]) == pytest.approx(5.0 + math.log(z), abs=1e-15)
    assert 5.0 + math.log(z) == pytest.approx(5.18518, abs=1e-5)


def test_worked_example_erratum_recorded(oracle_lib):
    """The printed entries 1, 2, 4 are a misprint; record how they arise, do not assert them."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    y, tr = oracle.softmax_online(g["scores"], g["block"])
    printed = g["printed"]["final_softmax"]
    for i in (0, 1, 3):
        assert abs(y[i] - printed[i]) > 0.005  # well beyond 3-decimal rounding: a misprint
    w1 = tr["carried"][1] / tr["run_l"][1]  # whole rebased block-1 weight
    assert w1 == pytest.approx(printed[0], abs=5e-4)
    assert w1 * math.exp(-1) == pytest.approx(printed[1], abs=5e-4)
    assert 1 - printed[0] - printed[1] - printed[2] == pytest.approx(printed[3], abs=1e-12)


# ---------------------------------------------------------------------------
# P6 — the invariant d_j = sum_{k<=j} exp(x_k - m_j) ("Online Softmax")
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("block", [1, 3, 4])
def test_online_invariant_every_step(oracle_lib, block):
    x = _rng(7).standard_normal(10) * 5  # the course file's demo shape: 10 values * 5
    y, tr = oracle.softmax_online(x, block)
    for b in range(len(tr["run_m"])):
        seen = x[: min((b + 1) * block, len(x))]
        assert tr["run_m"][b] == max(seen)
        direct = math.fsum(math.exp(v - tr["run_m"][b]) for v in seen)
        assert tr["run_l"][b] == pytest.approx(direct, rel=1e-14)
    ref = np.exp(x - x.max()) / math.fsum(np.exp(x - x.max()))
    np.testing.assert_allclose(y, ref, rtol=1e-14)


def test_online_leading_neg_inf_block(oracle_lib):
    """A block of -inf at the start carries nothing ((-inf) - (-inf) never evaluated)."""
    y, tr = oracle.softmax_online([-np.inf, -np.inf, 1.0, 2.0], 2)
    assert tr["run_m"][0] == -np.inf and tr["run_l"][0] == 0.0
    np.testing.assert_allclose(y, [0, 0, 1 / (1 + math.e), math.e / (1 + math.e)], rtol=1e-15)


# ---------------------------------------------------------------------------
# P2 — L = m + ln l is the logsumexp of the scaled, masked scores
# ---------------------------------------------------------------------------

def test_lse_identity_against_scipy(oracle_lib):
    from scipy.special import logsumexp
    rng = _rng(11)
    for causal in (False, True):
        n, d = 97, 32
        q, k, v = (rng.standard_normal((n, d)) * 2 for _ in range(3))
        scale = 1 / math.sqrt(d)
        o, lse = oracle.attention_f64(q, k, v, causal, scale)
        s = (q @ k.T) * scale
        if causal:
            s = np.where(np.triu(np.ones((n, n), bool), 1), -np.inf, s)
        np.testing.assert_allclose(lse, logsumexp(s, axis=1), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# library pin — torch's own attention on the CPU in fp64
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nq,nk,d,causal", [(64, 64, 16, False), (64, 64, 16, True),
                                             (33, 70, 8, False), (70, 33, 8, True),
                                             (5, 129, 64, False)])
def test_part1_matches_torch_sdpa(oracle_lib, nq, nk, d, causal):
    import torch
    rng = _rng(nq * 1000 + nk + d)
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    scale = 0.37
    o, _ = oracle.attention_f64(q, k, v, causal, scale)
    mask = None
    if causal:  # key kk visible to query r iff kk <= r (top-left)
        mask = torch.from_numpy(np.arange(nk)[None, :] <= np.arange(nq)[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=mask, scale=scale)[0].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# P5 — closed-form special cases
# ---------------------------------------------------------------------------

def test_special_single_key(oracle_lib):
    rng = _rng(1)
    q, k, v = rng.standard_normal((5, 8)), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    o, lse = oracle.attention_f64(q, k, v, False, 0.5)
    np.testing.assert_array_equal(o, np.repeat(v, 5, axis=0))
    np.testing.assert_allclose(lse, 0.5 * (q @ k[0]), rtol=1e-15)


def test_special_zero_queries_average_visible_values(oracle_lib):
    rng = _rng(2)
    n, d = 12, 6
    q = np.zeros((n, d))
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    for causal in (False, True):
        o, lse = oracle.attention_f64(q, k, v, causal, 1.0)
        for r in range(n):
            vis = r + 1 if causal else n
            np.testing.assert_allclose(o[r], v[:vis].mean(axis=0), rtol=1e-13, atol=1e-15)
            assert lse[r] == pytest.approx(math.log(vis), rel=1e-15)


def test_special_causal_row_zero(oracle_lib):
    rng = _rng(3)
    q, k, v = (rng.standard_normal((9, 5)) for _ in range(3))
    o, lse = oracle.attention_f64(q, k, v, True, 0.25)
    np.testing.assert_array_equal(o[0], v[0])
    assert lse[0] == pytest.approx(0.25 * float(q[0] @ k[0]), rel=1e-15)


def test_special_constant_values(oracle_lib):
    rng = _rng(4)
    q, k = rng.standard_normal((7, 4)), rng.standard_normal((11, 4))
    c = np.array([1.5, -2.0, 0.25, 3.0])
    v = np.tile(c, (11, 1))
    o, _ = oracle.attention_f64(q, k, v, False, 1.0)
    np.testing.assert_allclose(o, np.tile(c, (7, 1)), rtol=1e-14)


def test_special_shift_invariance(oracle_lib):
    """Adding a constant to every logit of a row leaves O and shifts L by it."""
    rng = _rng(5)
    n, d, a, scale = 10, 6, 3.7, 0.5
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    q2 = np.concatenate([q, np.full((n, 1), a)], axis=1)  # extra component a ...
    k2 = np.concatenate([k, np.ones((n, 1))], axis=1)     # ... against 1: logit += scale*a
    v2 = np.concatenate([v, np.zeros((n, 1))], axis=1)    # same head size for q, k, v
    for causal in (False, True):
        o1, l1 = oracle.attention_f64(q, k, v, causal, scale)
        o2, l2 = oracle.attention_f64(q2, k2, v2, causal, scale)
        np.testing.assert_allclose(o2[:, :d], o1, rtol=1e-13, atol=1e-14)
        assert not o2[:, d].any()
        np.testing.assert_allclose(l2 - l1, scale * a, rtol=1e-12)


def test_special_dominant_key(oracle_lib):
    rng = _rng(6)
    n, d = 16, 4
    k, v = rng.standard_normal((n, d)) * 0.1, rng.standard_normal((n, d))
    k[9] = [60.0, 0, 0, 0]
    q = np.tile([1.0, 0, 0, 0], (3, 1))
    o, _ = oracle.attention_f64(q, k, v, False, 1.0)
    assert np.abs(o - v[9]).max() < 1e-20 + n * math.exp(-59) * np.abs(v).max()


# ---------------------------------------------------------------------------
# P3 — (+) is associative and commutative and folds to the definition
# ---------------------------------------------------------------------------

def _leaves(q_row, k, v, scale, visible):
    return [oracle.leaf_state(scale * float(q_row @ k[j]), v[j]) for j in range(visible)]


def _fold(states):
    acc = oracle.empty_state(states[0].size - 2)
    for s in states:
        acc = oracle.merge(acc, s)
    return acc


def _tree(states, rng):
    states = list(states)
    while len(states) > 1:
        i = int(rng.integers(0, len(states) - 1))
        states[i:i + 2] = [oracle.merge(states[i], states[i + 1])]
    return states[0]


@pytest.mark.parametrize("nk,d,sigma", [(40, 8, 1.0), (257, 32, 3.0), (600, 128, 3.0)])
def test_merge_laws_random_partitions(oracle_lib, nk, d, sigma):
    rng = _rng(nk + d)
    q = rng.standard_normal((3, d)) * sigma
    k = rng.standard_normal((nk, d)) * sigma
    v = rng.standard_normal((nk, d))
    scale = 1 / math.sqrt(d)  # logits of std ~ sigma^2 (up to 9)
    o_ref, l_ref = oracle.attention_f64(q, k, v, False, scale)
    vmax = np.abs(v).max()
    for r in range(3):
        leaves = _leaves(q[r], k, v, scale, nk)
        cuts = np.sort(rng.choice(np.arange(1, nk), size=int(rng.integers(0, min(nk - 1, 12))),
                                  replace=False))
        blocks = [_fold(leaves[a:b]) for a, b in zip([0, *cuts], [*cuts, nk])]
        for st in (_fold(blocks), _tree(blocks, rng),
                   _fold([blocks[i] for i in rng.permutation(len(blocks))]),
                   _tree([leaves[i] for i in rng.permutation(nk)], rng)):
            o = st[2:] / st[1]
            lse = st[0] + math.log(st[1])
            assert np.abs(o - o_ref[r]).max() <= 1e-12 * vmax
            assert abs(lse - l_ref[r]) <= 1e-12 * max(1.0, abs(l_ref[r]))


def test_merge_identity_and_symmetry(oracle_lib):
    rng = _rng(8)
    a = np.concatenate([[0.3, 2.5], rng.standard_normal(4)])
    b = np.concatenate([[-1.2, 0.7], rng.standard_normal(4)])
    e = oracle.empty_state(4)
    np.testing.assert_array_equal(oracle.merge(a, e), a)
    np.testing.assert_array_equal(oracle.merge(e, a), a)
    np.testing.assert_allclose(oracle.merge(a, b), oracle.merge(b, a), rtol=1e-15)
    ab = oracle.merge(a, b)
    # closed form of the merge: max, then both terms rebased to it
    m = max(a[0], b[0])
    assert ab[0] == m
    assert ab[1] == pytest.approx(a[1] * math.exp(a[0] - m) + b[1] * math.exp(b[0] - m), rel=1e-15)


# ---------------------------------------------------------------------------
# P8 — part 2 (scalar online accumulator, any key blocking) agrees with part 1
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("key_block", [0, 1, 7, 64, 1000])
def test_part2_matches_part1(oracle_lib, causal, key_block):
    rng = _rng(21 + key_block)
    n, d = 150, 64
    q, k = rng.standard_normal((n, d)) * 3, rng.standard_normal((n, d)) * 3
    v = rng.standard_normal((n, d))
    scale = 1 / 8
    o1, l1 = oracle.attention_f64(q, k, v, causal, scale)
    o2, l2, raised = oracle.online_f64(q, k, v, causal, scale, key_block)
    assert np.abs(o2 - o1).max() <= 1e-12 * np.abs(v).max()
    assert np.abs(l2 - l1).max() <= 1e-12 * max(1.0, np.abs(l1).max())
    if key_block in (0, 1):  # per-key running max raised at least once on most rows
        assert raised.mean() > 1.0


# ---------------------------------------------------------------------------
# raw-buffer entry points: widening of the stored dtypes
# ---------------------------------------------------------------------------

def test_raw_rows_widen_exactly(oracle_lib):
    from flashattention_tiling_online_amd import inputs
    w = inputs.custom("t", 2, 3, 40, 50, 16, "bf16", True, seed=77)
    q, k, v = inputs.make_qkv(w)
    sel_bh, sel_row = inputs.sample_rows(w, 6, 40)
    o, lse = oracle.ref_rows_f64(q, k, v, True, w.scale, "bf16", sel_bh, sel_row, threads=3)
    # the same values stored as fp32 (exact) give bit-identical results
    qq, kk, vv = (oracle.widen(a, "bf16").astype(np.float32) for a in (q, k, v))
    o2, l2 = oracle.ref_rows_f64(qq, kk, vv, True, w.scale, "f32", sel_bh, sel_row)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(l2, lse)
    # fp16 storage, including subnormals, widens exactly
    wf = inputs.custom("t16", 1, 2, 30, 30, 16, "f16", False, seed=78, sigma_q=1e-5)
    qf, kf, vf = inputs.make_qkv(wf)
    assert (np.abs(qf) < np.float16(6.1e-5)).any()  # subnormal inputs present
    bh = np.repeat(np.arange(2), 30)
    rows = np.tile(np.arange(30), 2)
    o4, l4 = oracle.ref_rows_f64(qf, kf, vf, False, wf.scale, "f16", bh, rows)
    for hd in range(2):
        o5, l5 = oracle.attention_f64(qf[0, hd].astype(np.float64), kf[0, hd].astype(np.float64),
                                      vf[0, hd].astype(np.float64), False, wf.scale)
        np.testing.assert_array_equal(o5, o4[bh == hd])
        np.testing.assert_array_equal(l5, l4[bh == hd])
    # per-head comparison with the fp64 one-head entry point
    for hd in np.unique(sel_bh):
        b, h = divmod(int(hd), w.H)
        rows = sel_row[sel_bh == hd]
        o3, l3 = oracle.attention_f64(oracle.widen(q[b, h], "bf16"), oracle.widen(k[b, h], "bf16"),
                                      oracle.widen(v[b, h], "bf16"), True, w.scale, rows)
        np.testing.assert_array_equal(o3, o[sel_bh == hd])
        np.testing.assert_array_equal(l3, lse[sel_bh == hd])


def test_fwd_ref_rounds_to_nearest_even(oracle_lib):
    from flashattention_tiling_online_amd import inputs
    for dt in ("bf16", "f16", "f32"):
        w = inputs.custom("t", 1, 2, 24, 30, 8, dt, False, seed=5)
        q, k, v = inputs.make_qkv(w)
        o, lse = oracle.fwd_ref(q, k, v, False, w.scale, dt)
        bh = np.repeat(np.arange(2), 24)
        rows = np.tile(np.arange(24), 2)
        o64, l64 = oracle.ref_rows_f64(q, k, v, False, w.scale, dt, bh, rows)
        np.testing.assert_array_equal(o.reshape(-1), oracle.round_to(o64, dt))
        np.testing.assert_array_equal(lse.reshape(-1), l64.astype(np.float32))


# ---------------------------------------------------------------------------
# rounding fp64 -> storage (used for fa_fwd_ref and by the input generator)
# ---------------------------------------------------------------------------

def _bf16_table():
    """All finite non-negative bf16 values, ascending, with their bit patterns."""
    bits = np.arange(0x7F81, dtype=np.uint32)  # +0 .. +inf (inf kept as the top sentinel)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return vals, bits.astype(np.uint16)


def _nearest_even_bf16(x, table):
    """Brute-force RNE: nearest table entry to |x|, ties to the even pattern, sign copied."""
    vals, bits = table
    a = np.abs(x)
    i = np.clip(np.searchsorted(vals, a), 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    dlo, dhi = a - lo, hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (bits[i] % 2 == 0))
    mag = np.where(pick_hi, bits[i], bits[i - 1])
    return (mag | np.where(np.signbit(x), 0x8000, 0)).astype(np.uint16)


def test_rounding_bf16_brute_force_and_generator(oracle_lib):
    from flashattention_tiling_online_amd import inputs
    rng = _rng(31)
    x = np.concatenate([rng.standard_normal(20000) * 3, rng.standard_normal(2000) * 1e-39,
                        [0.0, -0.0, 1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)]])
    table = _bf16_table()
    nz = x != 0
    want = _nearest_even_bf16(x[nz], table)
    got_oracle = oracle.round_to(x, "bf16")
    got_gen = inputs.round_fp64(x, "bf16")
    np.testing.assert_array_equal(got_oracle[nz], want)
    np.testing.assert_array_equal(got_gen, got_oracle)
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert got_oracle[-3] == 0x3F80 and got_oracle[-1] == 0xBF80
    assert got_oracle[-2] == 0x3F82  # 1 + 3*2^-8 -> 1 + 2^-6 (even mantissa)


def test_rounding_f16_f32_against_numpy(oracle_lib):
    from flashattention_tiling_online_amd import inputs
    rng = _rng(32)
    x = np.concatenate([rng.standard_normal(20000) * 100, rng.standard_normal(2000) * 1e-6,
                        [70000.0, 65519.99, 65520.0, -1e-8]])
    np.testing.assert_array_equal(oracle.round_to(x, "f16"), x.astype(np.float16))
    np.testing.assert_array_equal(inputs.round_fp64(x, "f16"), x.astype(np.float16))
    np.testing.assert_array_equal(oracle.round_to(x, "f32"), x.astype(np.float32))
