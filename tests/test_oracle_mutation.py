"""Mutation tests: the pins have teeth (CPU only).

Each case plants one plausible mistake in a private copy of the oracle's C
source — compiled into a temporary library, never touching the real one — and
checks that at least one pin of the battery below rejects it.  The first cases
are the blog/article's own troubleshooting entry (a rescale factor forgotten in
the running sum — "手写"/CUTLASS article section 3.3 and its section 6.3 table);
the rest are a dropped scale, an inverted mask, a wrong index, a wrong sign, and in
the gradients a dropped softmax-Jacobian term, a flipped sign, an unweighted D, a
dropped scale and wrong operands, and in dropout a broken generator round, an
inverted keep test, a dropped keep scale and the mask left out of dV or dP, and in
the caller masks a reversed bit order, an ignored mask, a wrong empty-row L and the
mask left out of the gradients.
"""
import json
import math
import os
import shutil

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SRC = os.path.join(os.path.dirname(oracle.__file__), "fa_oracle.c")

MUTANTS = {
    "softmax_sum_not_rebased": ("double carry = (l == 0.0) ? 0.0 : l * exp(m - m_new);",
                                "double carry = (l == 0.0) ? 0.0 : l;"),
    "online_rescale_dropped": ("double c = first ? 0.0 : exp(m_old - m_new);",
                               "double c = first ? 0.0 : 1.0;"),
    "online_output_not_rescaled": ("st[2 + t] = st[2 + t] * c + e * vrow[t];",
                                   "st[2 + t] = st[2 + t] + e * vrow[t];"),
    "merge_sum_not_rebased": ("double d = a[1] * ca + b[1] * cb;",
                              "double d = a[1] + b[1] * cb;"),
    "merge_wrong_sign": ("double cb = exp(mb - m);", "double cb = exp(m - mb);"),
    "scale_dropped": ("return scale * dot;", "return dot;"),
    "mask_inverted": ("if (causal && kk > r)", "if (causal && kk < r)"),
    "mask_off_by_one": ("if (causal && kk > r)", "if (causal && kk >= r)"),
    "value_index_transposed": ("o_row[t] += pk * v[kk * d + t];",
                               "o_row[t] += pk * v[kk * d + (d - 1 - t)];"),
    "lse_wrong_sign": ("*lse = m + log(l);", "*lse = m - log(l);"),
    "online_lse_wrong_sign": ("*lse = seen ? run[0] + log(run[1])", "*lse = seen ? run[0] - log(run[1])"),
    # gradients (part 3): the softmax-Jacobian term, signs, scales and operands
    "bwd_D_dropped": ("const double ds = p[kk] * (dp[kk] - D);",
                      "const double ds = p[kk] * dp[kk];"),
    "bwd_dS_wrong_sign": ("const double ds = p[kk] * (dp[kk] - D);",
                          "const double ds = p[kk] * (D - dp[kk]);"),
    "bwd_D_not_weighted": ("D += p[kk] * dp[kk];", "D += dp[kk];"),
    "bwd_dq_scale_dropped": ("dq[r * d + t] += scale * ds * k[kk * d + t];",
                             "dq[r * d + t] += ds * k[kk * d + t];"),
    "bwd_dk_uses_k": ("dk[kk * d + t] += scale * ds * q_row[t];",
                      "dk[kk * d + t] += scale * ds * k[kk * d + t];"),
    "bwd_dv_uses_dp": ("dv[kk * d + t] += pz * do_row[t];",
                       "dv[kk * d + t] += dp[kk] * do_row[t];"),
    # dropout (part 4): the generator, the keep test, the scale, the mask's two uses
    "philox_key_dropped": ("(uint32_t)(p1 >> 32) ^ c[1] ^ k0;", "(uint32_t)(p1 >> 32) ^ c[1];"),
    "dropout_compare_inverted": ("return (int)byte < dr->t ? 0.0 : dr->keep_scale;",
                                 "return (int)byte >= dr->t ? 0.0 : dr->keep_scale;"),
    "dropout_scale_dropped": ("dr->keep_scale = 256.0 / (256.0 - (double)t);",
                              "dr->keep_scale = 1.0;"),
    "dropout_dv_unmasked": ("const double pz = p[kk] * drop_factor(dr, r, kk);",
                            "const double pz = p[kk];"),
    "dropout_dp_unmasked": ("dp[kk] = acc * drop_factor(dr, r, kk);", "dp[kk] = acc;"),
    # caller masks (part 5): the bit order, the mask left out, the empty-row reading,
    # the mask left out of the backward
    "mask_bit_order_reversed": ("((mrow[kk / 32] >> (kk % 32)) & 1u)",
                                "((mrow[kk / 32] >> (31 - kk % 32)) & 1u)"),
    "mask_ignored": ("return !mrow || ((mrow[kk / 32] >> (kk % 32)) & 1u);", "return 1;"),
    "empty_row_lse_zero": ("        *lse = -INFINITY;\n        return;",
                           "        *lse = 0.0;\n        return;"),
    "bwd_mask_dropped": ("mask_rows ? mask_rows + r * W : NULL", "NULL"),
}


def _pins(L):
    """Run the pin battery against library L; return the names of the pins that fail."""
    failed = []

    def check(name, fn):
        try:
            fn()
        except (AssertionError, oracle.OracleError, FloatingPointError, ValueError):
            failed.append(name)

    def worked_example():
        g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
        y, tr = oracle.softmax_online(g["scores"], g["block"], L=L)
        z = math.fsum(math.exp(v - 5.0) for v in g["scores"])
        assert abs(tr["run_l"][1] - g["printed"]["total_sum"]) < 6e-4
        np.testing.assert_allclose(y, [math.exp(v - 5.0) / z for v in g["scores"]], rtol=1e-14)

    def torch_sdpa():
        import torch
        rng = np.random.default_rng(3)
        for causal in (False, True):
            q, k, v = (rng.standard_normal((24, 8)) for _ in range(3))
            o, _ = oracle.attention_f64(q, k, v, causal, 0.4, L=L)
            mask = torch.from_numpy(np.tril(np.ones((24, 24), bool))) if causal else None
            ref = torch.nn.functional.scaled_dot_product_attention(
                *(torch.from_numpy(a)[None] for a in (q, k, v)), attn_mask=mask, scale=0.4)[0]
            np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)

    def lse_scipy():
        from scipy.special import logsumexp
        rng = np.random.default_rng(4)
        q, k, v = (rng.standard_normal((20, 8)) for _ in range(3))
        _, lse = oracle.attention_f64(q, k, v, False, 0.4, L=L)
        np.testing.assert_allclose(lse, logsumexp(0.4 * q @ k.T, axis=1), rtol=1e-13)

    def part2_vs_part1():
        rng = np.random.default_rng(5)
        q, k = rng.standard_normal((30, 16)) * 3, rng.standard_normal((30, 16)) * 3
        v = rng.standard_normal((30, 16))
        for causal in (False, True):
            o1, l1 = oracle.attention_f64(q, k, v, causal, 0.25, L=L)
            for kb in (0, 5):
                o2, l2, _ = oracle.online_f64(q, k, v, causal, 0.25, kb, L=L)
                np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)

    def merge_closed_form():
        a = np.array([0.3, 2.5, 1.0, -2.0])
        b = np.array([-1.2, 0.7, 0.5, 4.0])
        ab = oracle.merge(a, b, L=L)
        m = 0.3
        ca, cb = 1.0, math.exp(-1.5)
        np.testing.assert_allclose(ab, [m, 2.5 * ca + 0.7 * cb, 1.0 * ca + 0.5 * cb,
                                        -2.0 * ca + 4.0 * cb], rtol=1e-15)

    def bwd_finite_differences():
        rng = np.random.default_rng(6)
        q, k, v, dout = (rng.standard_normal((4, 3)) for _ in range(4))
        for causal in (False, True):
            got = oracle.attention_bwd_f64(q, k, v, dout, causal, 0.6, L=L)
            h = 1e-5
            for which in range(3):
                for idx in np.ndindex(4, 3):
                    args = [q.copy(), k.copy(), v.copy()]
                    args[which][idx] += h
                    up = np.sum(dout * oracle.attention_f64(*args, causal, 0.6, L=L)[0])
                    args[which][idx] -= 2 * h
                    dn = np.sum(dout * oracle.attention_f64(*args, causal, 0.6, L=L)[0])
                    assert abs((up - dn) / (2 * h) - got[which][idx]) < 1e-7

    def bwd_torch_autograd():
        import torch
        rng = np.random.default_rng(8)
        q, k, v, dout = (rng.standard_normal((12, 4)) for _ in range(4))
        t = [torch.from_numpy(a).clone().requires_grad_(True) for a in (q, k, v)]
        torch.nn.functional.scaled_dot_product_attention(
            *(x[None] for x in t), scale=0.5)[0].backward(torch.from_numpy(dout))
        got = oracle.attention_bwd_f64(q, k, v, dout, False, 0.5, L=L)
        for g, x in zip(got, t):
            np.testing.assert_allclose(g, x.grad.numpy(), rtol=1e-10, atol=1e-12)

    def philox_kat():
        g = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
        for vec in g["vectors"]:
            got = oracle.philox4x32_10([int(x, 16) for x in vec["ctr"]],
                                       [int(x, 16) for x in vec["key"]], L=L)
            assert got == [int(x, 16) for x in vec["out"]]

    def dropout_unbiased():
        keep = oracle.dropout_keep(77, 64, 1, 256, 256, L=L).astype(np.float64)
        assert abs(keep.mean() - 0.75) < 0.01
        rng = np.random.default_rng(9)
        q, k, v = (rng.standard_normal((64, 4)) for _ in range(3))
        v[:] = 1.0  # O = sum_j P_j Z_j: its mean over rows is E[Z] = 1
        o, _ = oracle.attention_dropout_f64(q, k, v, False, 0.0001, 64, 5, L=L)
        assert abs(o.mean() - 1.0) < 0.05

    def dropout_finite_differences():
        rng = np.random.default_rng(10)
        q, k, v, dout = (rng.standard_normal((4, 3)) for _ in range(4))
        got = oracle.attention_bwd_dropout_f64(q, k, v, dout, False, 0.6, 90, 3, 0, L=L)
        h = 1e-5
        for which in range(3):
            for idx in np.ndindex(4, 3):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += h
                up = np.sum(dout * oracle.attention_dropout_f64(*args, False, 0.6, 90, 3, L=L)[0])
                args[which][idx] -= 2 * h
                dn = np.sum(dout * oracle.attention_dropout_f64(*args, False, 0.6, 90, 3, L=L)[0])
                assert abs((up - dn) / (2 * h) - got[which][idx]) < 1e-7

    def masked_torch_sdpa():
        import torch
        from flashattention_tiling_online_amd import inputs
        rng = np.random.default_rng(11)
        q, k, v = (rng.standard_normal((20, 8)) for _ in range(3))
        k, v = rng.standard_normal((45, 8)), rng.standard_normal((45, 8))
        vis = rng.random((20, 45)) < 0.5
        vis[4] = False
        live = vis.any(axis=1)
        o, lse = oracle.attention_masked_f64(q, k, v, inputs.pack_mask(vis), False, 0.4, L=L)
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(a)[None] for a in (q, k, v)),
            attn_mask=torch.from_numpy(vis)[None], scale=0.4)[0].numpy()
        np.testing.assert_allclose(o[live], ref[live], rtol=1e-12, atol=1e-13)
        assert (o[~live] == 0).all() and np.isneginf(lse[~live]).all()

    def masked_bwd_torch():
        import torch
        from flashattention_tiling_online_amd import inputs
        rng = np.random.default_rng(12)
        q, dout = rng.standard_normal((10, 4)), rng.standard_normal((10, 4))
        k, v = rng.standard_normal((37, 4)), rng.standard_normal((37, 4))
        vis = rng.random((10, 37)) < 0.5
        vis[:, 0] = True
        got = oracle.attention_bwd_masked_f64(q, k, v, dout, inputs.pack_mask(vis), False, 0.5,
                                              L=L)
        t = [torch.from_numpy(a).clone().requires_grad_(True) for a in (q, k, v)]
        torch.nn.functional.scaled_dot_product_attention(
            *(x[None] for x in t), attn_mask=torch.from_numpy(vis)[None],
            scale=0.5)[0].backward(torch.from_numpy(dout))
        for g, x in zip(got, t):
            np.testing.assert_allclose(g, x.grad.numpy(), rtol=1e-10, atol=1e-12)

    for name, fn in [("worked_example", worked_example), ("torch_sdpa", torch_sdpa),
                     ("masked_torch_sdpa", masked_torch_sdpa),
                     ("masked_bwd_torch", masked_bwd_torch),
                     ("lse_scipy", lse_scipy), ("part2_vs_part1", part2_vs_part1),
                     ("merge_closed_form", merge_closed_form),
                     ("bwd_finite_differences", bwd_finite_differences),
                     ("bwd_torch_autograd", bwd_torch_autograd), ("philox_kat", philox_kat),
                     ("dropout_unbiased", dropout_unbiased),
                     ("dropout_finite_differences", dropout_finite_differences)]:
        check(name, fn)
    return failed


def test_unmutated_oracle_passes_battery(oracle_lib):
    assert _pins(oracle_lib) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(before, after)
    cdir = tmp_path / "oracle"
    cdir.mkdir()
    (cdir / "fa_oracle.c").write_text(mutated)
    inc = tmp_path / "include"
    inc.mkdir()
    shutil.copy(os.path.join(os.path.dirname(SRC), "..", "include", "fa_oracle.h"), inc)
    so = str(tmp_path / "libmutant.so")
    oracle.build(so, str(cdir / "fa_oracle.c"))
    L = oracle.load(so)
    with np.errstate(all="ignore"):
        failed = _pins(L)
    assert failed, f"mutant {name} passed every pin"
