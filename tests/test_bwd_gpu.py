"""GPU parity of the backward pass (fa_bwd, through the C-ABI) against the fp64 oracle.

The GPU forward (fa_fwd) produces O and L, the GPU backward the gradients from them;
the oracle (part 3) computes the gradients of sum(dO o O) from Q, K, V and dO alone,
in fp64.  The pages state no tolerance for the gradients; the bound follows from the
arithmetic of the GPU path and is applied to every element (tests/bwd_bounds.py):
|G_gpu - G_ref| <= C u (|G_ref| + A), u the unit roundoff of the input dtype and A the
sum of the magnitudes of the products that make up that element of the gradient.

Besides parity on all rows of small shapes and on seeded samples of rows (dQ) and
keys (dK, dV) of the large workloads: invariants at any size (sum_j dK_j = 0 and
sum_j dV_j = sum_i dO_i per head, up to the same rounding), Nq = 0 (dK = dV = 0),
determinism, and argument errors.
"""
import numpy as np
import pytest

import oracle
from flashattention_tiling_online_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import flashattention_tiling_online_amd as fa  # noqa: E402
import bwd_bounds  # noqa: E402
from parity_util import DEV, say, to_dev, to_host  # noqa: E402

# norm-wise slack of the invariants below (sums of many rounded terms)
BOUND = {"bf16": (2e-2, 5e-2), "f16": (3e-3, 1e-2)}


def run_bwd(w, q, k, v, dout):
    tq, tk, tv, tdo = (to_dev(a, w.dtype) for a in (q, k, v, dout))
    o, lse = fa.fa_fwd(tq, tk, tv, causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.fa_bwd(tq, tk, tv, o, lse, tdo, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_all_rows(w):
    say(f"[bwd] {w.describe()}")
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_do(w)
    dq, dk, dv = run_bwd(w, q, k, v, dout)
    g = [oracle.widen(to_host(t, w.dtype), w.dtype).reshape(w.B * w.H, -1, w.d)
         for t in (dq, dk, dv)]
    for bh in range(w.B * w.H):
        ref = oracle.bwd_head_f64(q, k, v, dout, w.causal, w.scale, w.dtype, bh)
        a = bwd_bounds.scales(w, q, k, v, dout, bh)
        say(f"  head {bh}")
        for name, got, r, s in zip(("dq", "dk", "dv"), g, ref, a):
            bwd_bounds.check(name, got[bh], r, s, w.dtype, say)
    return q, k, v, dout, dq, dk, dv


SMALL = [
    ("bwd_tiny", 1, 1, 1, 1, 128, "bf16", False, 51),
    ("bwd_128", 1, 2, 128, 128, 128, "bf16", False, 52),
    ("bwd_128_causal", 1, 2, 128, 128, 128, "bf16", True, 53),
    ("bwd_ragged_causal", 2, 1, 200, 333, 64, "bf16", True, 54),
    ("bwd_ragged_d128", 1, 2, 257, 190, 128, "f16", False, 55),
    ("bwd_nq_gt_nk_causal", 1, 2, 300, 100, 128, "bf16", True, 56),
    ("bwd_f16_causal_d64", 1, 3, 321, 321, 64, "f16", True, 57),
    ("bwd_large_logits", 1, 2, 256, 512, 128, "bf16", True, 58, 3.0),
    # causal grids of whole heads per XCD (16 heads: items listed by weight across the
    # XCD's heads) and of split heads (12 heads: head-major order kept)
    ("bwd_16h_causal_order", 2, 8, 300, 300, 128, "bf16", True, 59),
    ("bwd_12h_causal_order", 1, 12, 260, 260, 128, "f16", True, 60),
]


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_bwd_all_rows(spec):
    name, B, H, Nq, Nk, d, dt, causal, seed, *sig = spec
    s = sig[0] if sig else 1.0
    w = inputs.custom(name, B, H, Nq, Nk, d, dt, causal, seed, sigma_q=s, sigma_k=s)
    check_all_rows(w)


@pytest.mark.parametrize("name", ["mh_d64", "mh_d64_causal"])
def test_bwd_small_workloads(name):
    w = inputs.WORKLOADS[name]
    q, k, v, dout, dq, dk, dv = check_all_rows(w)
    invariants(w, dout, dk, dv)


def invariants(w, dout, dk, dv):
    """Per head: sum over keys of dK is 0 and of dV is sum over queries of dO (each row
    of dS sums to 0, each row of P to 1), up to the rounding bound."""
    cf, _ = BOUND[w.dtype]
    dkf = dk.float().reshape(w.B * w.H, w.Nk, w.d)
    dvf = dv.float().reshape(w.B * w.H, w.Nk, w.d)
    dof = to_dev(dout, w.dtype).float().reshape(w.B * w.H, w.Nq, w.d)
    s_dk = dkf.sum(dim=1)
    s_dv = dvf.sum(dim=1)
    s_do = dof.sum(dim=1)
    # sums of n rounded terms: allow cf times the norm of the terms being summed
    tol_k = cf * dkf.abs().sum(dim=1) + 1e-6
    tol_v = cf * dvf.abs().sum(dim=1) + 1e-6
    assert bool((s_dk.abs() <= tol_k).all())
    assert bool(((s_dv - s_do).abs() <= tol_v).all())


@pytest.mark.parametrize("name", ["long_4k", "self_8k_causal", "cross_1k_8k"])
def test_bwd_sampled(name):
    w = inputs.WORKLOADS[name]
    say(f"[bwd sampled] {w.describe()}")
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_do(w)
    dq, dk, dv = run_bwd(w, q, k, v, dout)
    sel_bh, sel_row = inputs.sample_rows(w, 2, 128)
    dq_ref = oracle.bwd_dq_rows_f64(q, k, v, dout, w.causal, w.scale, w.dtype, sel_bh, sel_row)
    dq_np = oracle.widen(to_host(dq, w.dtype), w.dtype).reshape(-1, w.d)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([inputs.SAMPLE_SEED, 7])))
    keys = np.sort(rng.choice(w.Nk, size=96, replace=False)).astype(np.int64)
    heads = np.unique(sel_bh)
    kb = np.repeat(heads, keys.size)
    kk = np.tile(keys, heads.size)
    dk_ref, dv_ref = oracle.bwd_dkv_keys_f64(q, k, v, dout, w.causal, w.scale, w.dtype, kb, kk)
    dk_np = oracle.widen(to_host(dk, w.dtype), w.dtype).reshape(-1, w.d)
    dv_np = oracle.widen(to_host(dv, w.dtype), w.dtype).reshape(-1, w.d)
    for h in heads:
        rows = sel_row[sel_bh == h]
        a_q, a_k, a_v = bwd_bounds.scales(w, q, k, v, dout, h, q_rows=rows, k_cols=keys)
        say(f"  head {h}")
        bwd_bounds.check("dq rows", dq_np[h * w.Nq + rows], dq_ref[sel_bh == h], a_q, w.dtype,
                         say)
        bwd_bounds.check("dk keys", dk_np[h * w.Nk + keys], dk_ref[kb == h], a_k, w.dtype, say)
        bwd_bounds.check("dv keys", dv_np[h * w.Nk + keys], dv_ref[kb == h], a_v, w.dtype, say)
    invariants(w, dout, dk, dv)


def test_bwd_no_queries_gives_zero_key_gradients():
    w = inputs.custom("bwd_nq0", 1, 2, 0, 100, 64, "bf16", False, 61)
    k, v = (to_dev(inputs.make_tensor(w, t), "bf16") for t in ("k", "v"))
    q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, 2, 0), dtype=torch.float32, device=DEV)
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(v, 7.0)
    fa.fa_bwd(q, k, v, q, lse, q, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert bool((dk == 0).all()) and bool((dv == 0).all())


def test_bwd_deterministic():
    w = inputs.custom("bwd_det", 2, 2, 384, 640, 128, "bf16", True, 62)
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_do(w)
    a = run_bwd(w, q, k, v, dout)
    b = run_bwd(w, q, k, v, dout)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bwd_invalid_arguments_raise():
    w = inputs.custom("bwd_bad", 1, 1, 64, 64, 64, "f32", False, 63)
    q, k, v = (to_dev(a, "f32") for a in inputs.make_qkv(w))
    lse = torch.zeros((1, 1, 64), device=DEV)
    with pytest.raises(fa.FAError):
        fa.fa_bwd(q, k, v, q, lse, q)  # fp32: unsupported
    qb = q.to(torch.bfloat16)
    with pytest.raises(fa.FAError):
        fa.fa_bwd(qb, k.to(torch.bfloat16), v.to(torch.bfloat16), qb, lse, qb, scale=-1.0)
    torch.cuda.synchronize()
