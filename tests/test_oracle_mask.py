"""Pins of the oracle's caller masks (part 5), CPU only.

The blog page "Flash Attention" (Algorithm 2) applies mask(S) to the scaled scores
before the softmax, and its Algorithm 4 recomputes P from the same masked scores in
the backward pass.  The oracle reads mask(S) as S[q, k] = -inf where the caller's
boolean mask is false, the mask bit-packed per query row (key k in bit k % 32 of word
k // 32); a row with no visible key gives O = 0, L = -inf and no gradient.  These
tests pin that against what does not come from the oracle:

* torch's fp64 CPU scaled_dot_product_attention with a boolean attn_mask (forward and
  autograd gradients) on rows that see at least one key;
* special cases with closed forms or exact equivalents: an all-visible mask is the
  unmasked oracle, a lower-triangular mask is the causal flag, a key-padding mask is
  attention over the first n keys, a row with one visible key returns that key's V;
* invariants: permuting the keys together with the mask's columns, and the online
  accumulator (part 2) over any key blocking, reproduce part 1;
* central finite differences of the masked forward for the masked gradients;
* the raw-buffer forms with a mask shared over batch and heads equal the per-head
  forms, and the rows with no visible key return exactly (0, -inf).
"""
import numpy as np
import pytest

import oracle
from flashattention_tiling_online_amd import inputs

torch = pytest.importorskip("torch")


def _rand(rng, *shape, sigma=1.0):
    return rng.standard_normal(shape) * sigma


def _torch_sdpa(q, k, v, vis, scale):
    return torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a)[None] for a in (q, k, v)),
        attn_mask=torch.from_numpy(vis)[None], scale=scale)[0].numpy()


@pytest.mark.parametrize("kind", ["random", "sliding_window", "block", "empty_rows"])
@pytest.mark.parametrize("nq,nk", [(37, 53), (64, 200), (5, 1)])
def test_masked_forward_equals_torch_sdpa(kind, nq, nk):
    rng = np.random.default_rng(nq * 1000 + nk)
    q, k, v = _rand(rng, nq, 16, sigma=2.0), _rand(rng, nk, 16, sigma=2.0), _rand(rng, nk, 16)
    vis = inputs.make_mask(kind, 1, 1, nq, nk, seed=nq + nk, window=7, tile=8)[0, 0]
    words = inputs.pack_mask(vis)
    o, lse = oracle.attention_masked_f64(q, k, v, words, False, 0.3)
    live = vis.any(axis=1)
    if live.any():
        ref = _torch_sdpa(q, k, v, vis, 0.3)
        np.testing.assert_allclose(o[live], ref[live], rtol=1e-12, atol=1e-13)
        s = 0.3 * q @ k.T
        from scipy.special import logsumexp
        np.testing.assert_allclose(lse[live], logsumexp(np.where(vis, s, -np.inf), axis=1)[live],
                                   rtol=1e-13, atol=1e-13)
    assert (o[~live] == 0.0).all() and np.isneginf(lse[~live]).all()


def test_all_visible_mask_is_the_unmasked_oracle():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 40, 8), _rand(rng, 70, 8), _rand(rng, 70, 8)
    words = inputs.pack_mask(np.ones((40, 70), bool))
    for causal in (False, True):
        a = oracle.attention_masked_f64(q, k, v, words, causal, 0.5)
        b = oracle.attention_f64(q, k, v, causal, 0.5)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_triangular_mask_is_the_causal_flag():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 50, 8), _rand(rng, 50, 8), _rand(rng, 50, 8)
    words = inputs.pack_mask(np.tril(np.ones((50, 50), bool)))
    a = oracle.attention_masked_f64(q, k, v, words, False, 0.5)
    b = oracle.attention_f64(q, k, v, True, 0.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_causal_flag_and_mask_combine():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 45, 8), _rand(rng, 45, 8), _rand(rng, 45, 8)
    vis = rng.random((45, 45)) < 0.6
    a = oracle.attention_masked_f64(q, k, v, inputs.pack_mask(vis), True, 0.5)
    b = oracle.attention_masked_f64(q, k, v, inputs.pack_mask(vis & np.tril(np.ones((45, 45),
                                                                                 bool))),
                                    False, 0.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_key_padding_is_attention_over_the_first_keys():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 30, 8), _rand(rng, 100, 8), _rand(rng, 100, 8)
    for n in (1, 31, 32, 33, 77):
        vis = np.zeros((30, 100), bool)
        vis[:, :n] = True
        a = oracle.attention_masked_f64(q, k, v, inputs.pack_mask(vis), False, 0.4)
        b = oracle.attention_f64(q, k[:n], v[:n], False, 0.4)
        np.testing.assert_allclose(a[0], b[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(a[1], b[1], rtol=1e-13, atol=1e-14)


def test_one_visible_key_returns_its_value():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 20, 8), _rand(rng, 90, 8), _rand(rng, 90, 8)
    pick = rng.integers(0, 90, size=20)
    vis = np.zeros((20, 90), bool)
    vis[np.arange(20), pick] = True
    o, lse = oracle.attention_masked_f64(q, k, v, inputs.pack_mask(vis), False, 0.4)
    np.testing.assert_allclose(o, v[pick], rtol=0, atol=0)
    np.testing.assert_allclose(lse, 0.4 * np.einsum("ij,ij->i", q, k[pick]), rtol=1e-14)


def test_key_permutation_invariance():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 25, 8, sigma=2), _rand(rng, 60, 8, sigma=2), _rand(rng, 60, 8)
    vis = rng.random((25, 60)) < 0.4
    perm = rng.permutation(60)
    a = oracle.attention_masked_f64(q, k, v, inputs.pack_mask(vis), False, 0.4)
    b = oracle.attention_masked_f64(q, k[perm], v[perm], inputs.pack_mask(vis[:, perm]), False,
                                    0.4)
    live = vis.any(axis=1)
    np.testing.assert_allclose(a[0][live], b[0][live], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(a[1][live], b[1][live], rtol=1e-13)


@pytest.mark.parametrize("kb", [0, 1, 7, 32, 64])
def test_online_part_equals_part_one(kb):
    rng = np.random.default_rng(7 + kb)
    q, k, v = _rand(rng, 33, 8, sigma=3), _rand(rng, 150, 8, sigma=3), _rand(rng, 150, 8)
    vis = inputs.make_mask("empty_rows", 1, 1, 33, 150, seed=kb)[0, 0]
    words = inputs.pack_mask(vis)
    for causal in (False, True):
        a = oracle.attention_masked_f64(q, k, v, words, causal, 0.3)
        b = oracle.online_masked_f64(q, k, v, words, causal, 0.3, kb)
        np.testing.assert_allclose(b[0], a[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(b[1], a[1], rtol=1e-12, atol=1e-12)
        dead = ~(vis & (np.tril(np.ones((33, 150), bool)) if causal else True)).any(axis=1)
        assert (b[0][dead] == 0).all() and np.isneginf(b[1][dead]).all()


def test_masked_gradients_equal_torch_autograd():
    rng = np.random.default_rng(8)
    q, k, v, dout = _rand(rng, 18, 4), _rand(rng, 23, 4), _rand(rng, 23, 4), _rand(rng, 18, 4)
    vis = rng.random((18, 23)) < 0.5
    vis[3] = False                      # a row with no visible key
    live = vis.any(axis=1)
    got = oracle.attention_bwd_masked_f64(q, k, v, dout, inputs.pack_mask(vis), False, 0.5)
    # torch on the live rows only (a row with no visible key has no softmax there)
    t = [torch.from_numpy(a).clone().requires_grad_(True) for a in (q[live], k, v)]
    out = torch.nn.functional.scaled_dot_product_attention(
        *(x[None] for x in t), attn_mask=torch.from_numpy(vis[live])[None], scale=0.5)[0]
    out.backward(torch.from_numpy(dout[live]))
    np.testing.assert_allclose(got[0][live], t[0].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got[1], t[1].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got[2], t[2].grad.numpy(), rtol=1e-10, atol=1e-12)
    assert (got[0][~live] == 0).all()


def test_masked_gradients_finite_differences():
    rng = np.random.default_rng(9)
    q, k, v, dout = (_rand(rng, 5, 3) for _ in range(4))
    vis = rng.random((5, 5)) < 0.6
    vis[:, 0] = True
    words = inputs.pack_mask(vis)
    for causal in (False, True):
        got = oracle.attention_bwd_masked_f64(q, k, v, dout, words, causal, 0.6)
        h = 1e-5
        for which in range(3):
            for idx in np.ndindex(5, 3):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += h
                up = np.sum(dout * oracle.attention_masked_f64(*args, words, causal, 0.6)[0])
                args[which][idx] -= 2 * h
                dn = np.sum(dout * oracle.attention_masked_f64(*args, words, causal, 0.6)[0])
                assert abs((up - dn) / (2 * h) - got[which][idx]) < 1e-7


@pytest.mark.parametrize("mb,mh", [(1, 1), (2, 1), (1, 3), (2, 3)])
def test_raw_forms_broadcast_the_mask(mb, mh):
    w = inputs.custom("mask_raw", 2, 3, 40, 70, 64, "bf16", False, seed=31)
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_do(w)
    vis = inputs.make_mask("empty_rows", mb, mh, 40, 70, seed=mb * 10 + mh)
    words = inputs.pack_mask(vis)
    sel_bh = np.repeat(np.arange(6), 40)
    sel_row = np.tile(np.arange(40), 6)
    o, lse = oracle.ref_rows_masked_f64(q, k, v, words, False, w.scale, "bf16", sel_bh, sel_row)
    o2, lse2 = oracle.ref_rows_masked_f64(q, k, v, words, False, w.scale, "bf16", sel_bh, sel_row,
                                          online_key_block=16)
    for bh in range(6):
        b, h = divmod(bh, 3)
        mrow = words[b if mb > 1 else 0, h if mh > 1 else 0]
        qh, kh, vh = (oracle.widen(a[b, h], "bf16") for a in (q, k, v))
        ref = oracle.attention_masked_f64(qh, kh, vh, mrow, False, w.scale)
        np.testing.assert_array_equal(o[bh * 40:(bh + 1) * 40], ref[0])
        np.testing.assert_array_equal(lse[bh * 40:(bh + 1) * 40], ref[1])
        np.testing.assert_allclose(o2[bh * 40:(bh + 1) * 40], ref[0], rtol=1e-12, atol=1e-12)
        g = oracle.bwd_head_masked_f64(q, k, v, dout, words, False, w.scale, "bf16", bh)
        gr = oracle.attention_bwd_masked_f64(qh, kh, vh, oracle.widen(dout[b, h], "bf16"), mrow,
                                             False, w.scale)
        for a_, b_ in zip(g, gr):
            np.testing.assert_array_equal(a_, b_)
