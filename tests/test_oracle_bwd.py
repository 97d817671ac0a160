"""Pins of the oracle's gradients (part 3), CPU only.

The oracle computes the gradients of sum(dO o O) by the plain definition the pages
give (course file flash_attention_backward; blog page Algorithm 4 and the
softmax-Jacobian derivation after it).  Nothing here re-types that formula; the
pins come from elsewhere:

* central finite differences of the forward oracle (part 1, separate code) — the
  gradients must be the derivative of the forward definition;
* torch's own fp64 CPU autograd of scaled_dot_product_attention — an independent
  implementation;
* algebra that holds for any inputs: sum_j dK_j = 0 (every row of dS sums to 0),
  sum_j dV_j = sum_i dO_i (every row of P sums to 1), dQ = dK = 0 when all value
  rows are equal, all gradients 0 when dO = 0, and the one-key closed form;
* the raw-buffer entry points (whole head, selected rows, selected keys, the
  rounded whole-tensor reference) agree with the fp64 one-head function.
"""
import numpy as np
import pytest

import oracle
from flashattention_tiling_online_amd import inputs


def _loss(q, k, v, dout, causal, scale):
    o, _ = oracle.attention_f64(q, k, v, causal, scale)
    return float(np.sum(dout * o))


def _numeric_grads(q, k, v, dout, causal, scale, h=1e-5):
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        for idx in np.ndindex(g.shape):
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (_loss(*plus, dout, causal, scale) - _loss(*minus, dout, causal, scale)) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("nq,nk,d,causal,sig", [
    (5, 6, 3, False, 1.0), (5, 6, 3, True, 1.0), (6, 4, 4, True, 1.5), (4, 7, 2, False, 2.0),
    (3, 3, 5, True, 0.5),
])
def test_bwd_is_the_derivative_of_the_forward(nq, nk, d, causal, sig):
    rng = np.random.default_rng(nq * 100 + nk * 10 + d + int(causal))
    q, k = rng.standard_normal((nq, d)) * sig, rng.standard_normal((nk, d)) * sig
    v, dout = rng.standard_normal((nk, d)), rng.standard_normal((nq, d))
    scale = 0.7
    got = oracle.attention_bwd_f64(q, k, v, dout, causal, scale)
    want = _numeric_grads(q, k, v, dout, causal, scale)
    for g, w, name in zip(got, want, ("dq", "dk", "dv")):
        np.testing.assert_allclose(g, w, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("nq,nk,d,causal", [(24, 24, 8, False), (24, 24, 8, True),
                                             (17, 40, 16, False), (30, 19, 4, True)])
def test_bwd_matches_torch_autograd(nq, nk, d, causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7 + nq + nk)
    q, k, v = (rng.standard_normal((n, d)) for n in (nq, nk, nk))
    dout = rng.standard_normal((nq, d))
    scale = 0.35
    tq, tk, tv = (torch.from_numpy(a).clone().requires_grad_(True) for a in (q, k, v))
    mask = torch.from_numpy(np.tril(np.ones((nq, nk), bool))) if causal else None
    o = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                                         attn_mask=mask, scale=scale)[0]
    o.backward(torch.from_numpy(dout))
    got = oracle.attention_bwd_f64(q, k, v, dout, causal, scale)
    for g, t, name in zip(got, (tq.grad, tk.grad, tv.grad), ("dq", "dk", "dv")):
        np.testing.assert_allclose(g, t.numpy(), rtol=1e-11, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_invariants(causal):
    rng = np.random.default_rng(11)
    nq, nk, d = 33, 29, 8
    q, k = rng.standard_normal((nq, d)) * 2, rng.standard_normal((nk, d)) * 2
    v, dout = rng.standard_normal((nk, d)), rng.standard_normal((nq, d))
    dq, dk, dv = oracle.attention_bwd_f64(q, k, v, dout, causal, 0.4)
    # every row of dS sums to zero -> the key gradients sum to zero
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    # every row of P sums to one -> the value gradients sum to the output gradients
    # (causal rows beyond the keys still see keys 0..nk-1; every row sees key 0)
    np.testing.assert_allclose(dv.sum(axis=0), dout.sum(axis=0), rtol=1e-12, atol=1e-12)
    # equal value rows: O does not depend on the scores -> no score gradients
    vc = np.tile(rng.standard_normal(d), (nk, 1))
    dq0, dk0, _ = oracle.attention_bwd_f64(q, k, vc, dout, causal, 0.4)
    assert np.abs(dq0).max() < 1e-12 and np.abs(dk0).max() < 1e-12
    # no output gradient -> no input gradient
    z = oracle.attention_bwd_f64(q, k, v, np.zeros_like(dout), causal, 0.4)
    assert all(np.abs(g).max() == 0 for g in z)
    # one key: P = 1 for every row -> dQ = dK = 0, dV = sum of dO
    dq1, dk1, dv1 = oracle.attention_bwd_f64(q, k[:1], v[:1], dout, causal, 0.4)
    assert np.abs(dq1).max() == 0 and np.abs(dk1).max() == 0
    np.testing.assert_allclose(dv1[0], dout.sum(axis=0), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("f16", False), ("f32", True)])
def test_bwd_raw_paths_agree(dtype, causal):
    w = inputs.custom("bwd_raw", 1, 2, 70, 90, 16, dtype, causal, 77)
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_do(w)
    L = oracle.lib()
    for bh in range(2):
        dq, dk, dv = oracle.bwd_head_f64(q, k, v, dout, causal, w.scale, dtype, bh)
        qw, kw, vw, dw = (oracle.widen(a, dtype).reshape(2, -1, 16)[bh] for a in (q, k, v, dout))
        e = oracle.attention_bwd_f64(qw, kw, vw, dw, causal, np.float64(np.float32(w.scale)), L=L)
        for a, b in zip((dq, dk, dv), e):
            assert np.array_equal(a, b)
        rows = np.arange(70)
        dq_r = oracle.bwd_dq_rows_f64(q, k, v, dout, causal, w.scale, dtype,
                                      np.full(70, bh), rows, threads=3)
        np.testing.assert_allclose(dq_r, dq, rtol=1e-12, atol=1e-13)
        keys = np.array([0, 5, 44, 89])
        dk_s, dv_s = oracle.bwd_dkv_keys_f64(q, k, v, dout, causal, w.scale, dtype,
                                             np.full(keys.size, bh), keys, threads=2)
        np.testing.assert_allclose(dk_s, dk[keys], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dv_s, dv[keys], rtol=1e-11, atol=1e-12)
    rq, rk, rv = oracle.bwd_ref(q, k, v, dout, causal, w.scale, dtype)
    dq, dk, dv = oracle.bwd_head_f64(q, k, v, dout, causal, w.scale, dtype, 1)
    assert np.array_equal(rq[0, 1], oracle.round_to(dq, dtype).reshape(70, 16))
    assert np.array_equal(rv[0, 1], oracle.round_to(dv, dtype).reshape(90, 16))
