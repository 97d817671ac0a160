"""GPU parity of dropout on P (fa_fwd_dropout, fa_bwd_dropout, through the C-ABI)
against the fp64 oracle (part 4).

Dropout follows the blog page's Algorithm 2 (P_dropped = dropout(P, p), O = P_dropped V,
L unchanged) and Algorithm 4 (the same Z regenerated for dV = P_dropped^T dO and
dS = P o (dP o Z - D)).  Z comes from Philox4x32-10 keyed by the seed, one call per
4x4 block of (query, key) elements, an element dropped iff its byte is below
t = round(256 p) (the reading documented in include/fa.h); both sides draw it, each
from its own implementation of the published generator.

Bounds.  The pages state none for dropout.  The GPU arithmetic is that of fa_fwd /
fa_bwd with the kept weights scaled by s = 256 / (256 - t), applied once in fp32, so
the forward bounds are fa_fwd's scaled by s plus the rounding of the output itself,
which dropout makes visible (s V is no longer a representable value even where one
key dominates): per element |dO| <= 1e-2 s + u |O_ref| and mean |dO| <= 1e-3 s +
u mean |O_ref|, with u = 2^-8 (bf16) or 2^-11 (fp16) the unit roundoff of the
output; |dL| <= 1e-3 (L does not see Z).  The gradient bounds are fa_bwd's relative
ones.

The keep decisions themselves are checked bit-exactly: with Q = 0 every visible key
has P = 1/n, and with V the identity (Nk <= d) O[q, k] is nonzero iff (q, k) is kept.
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



def threshold(p):
    return int(round(256 * p))


def keep_scale(p):
    return 256.0 / (256.0 - threshold(p))


def run_fwd(w, q, k, v, p, seed):
    tq, tk, tv = (to_dev(a, w.dtype) for a in (q, k, v))
    o, lse = fa.fa_fwd_dropout(tq, tk, tv, p, seed, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o, lse


def compare_fwd(w, p, o_np, lse_np, sel_bh, sel_row, o64, l64):
    s = keep_scale(p)
    u = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -11
    o_sel = oracle.widen(o_np.reshape(-1, w.d)[sel_bh * w.Nq + sel_row], w.dtype)
    l_sel = lse_np.reshape(-1)[sel_bh * w.Nq + sel_row].astype(np.float64)
    assert np.isfinite(o_sel).all() and np.isfinite(l_sel).all()
    err = np.abs(o_sel - o64)
    derr_l = np.abs(l_sel - l64)
    lim = 1e-2 * s + u * np.abs(o64)
    mean_lim = 1e-3 * s + u * np.abs(o64).mean()
    say(f"  {w.name} p={p}: max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} "
        f"(limit {mean_lim:.3e}) max|dL|={derr_l.max():.3e} max|dO|/limit={(err / lim).max():.3f}")
    assert (err <= lim).all(), f"max|dO|/limit {(err / lim).max():.3f}"
    assert err.mean() <= mean_lim
    assert derr_l.max() <= 1e-3


FWD_SHAPES = [
    # name, B, H, Nq, Nk, d, dtype, causal, seed
    ("drop_tiny", 1, 1, 1, 1, 128, "bf16", False, 71),
    ("drop_128", 1, 2, 128, 128, 128, "bf16", False, 72),
    ("drop_ragged_causal", 2, 3, 300, 300, 128, "bf16", True, 73),
    ("drop_rect_d64", 1, 4, 200, 333, 64, "f16", False, 74),
    ("drop_causal_d64", 2, 2, 257, 257, 64, "bf16", True, 75),
    ("drop_nq_gt_nk", 1, 2, 500, 129, 128, "f16", True, 76),
]


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
@pytest.mark.parametrize("spec", FWD_SHAPES, ids=[s[0] for s in FWD_SHAPES])
def test_dropout_fwd_all_rows(spec, p):
    name, B, H, Nq, Nk, d, dt, causal, seed = spec
    w = inputs.custom(name, B, H, Nq, Nk, d, dt, causal, seed)
    q, k, v = inputs.make_qkv(w)
    rng_seed = 0x5EED0000 + seed
    o, lse = run_fwd(w, q, k, v, p, rng_seed)
    sel_bh = np.repeat(np.arange(B * H), Nq)
    sel_row = np.tile(np.arange(Nq), B * H)
    o64, l64 = oracle.ref_rows_dropout_f64(q, k, v, causal, w.scale, dt, threshold(p), rng_seed,
                                           sel_bh, sel_row)
    compare_fwd(w, p, to_host(o, dt), lse.cpu().numpy(), sel_bh, sel_row, o64, l64)


@pytest.mark.parametrize("name", ["mh_d64", "mh_d64_causal", "self_8k_causal", "ctx_32k_causal"])
def test_dropout_fwd_workloads_sampled(name):
    w = inputs.WORKLOADS[name]
    p, seed = 0.1, 0xD0D0CAFEF00D
    say(f"[dropout] {w.describe()}")
    q, k, v = inputs.make_qkv(w)
    o, lse = run_fwd(w, q, k, v, p, seed)
    sel_bh, sel_row = inputs.sample_rows(w, 4, 256 if w.Nq > 1024 else w.Nq)
    o64, l64 = oracle.ref_rows_dropout_f64(q, k, v, w.causal, w.scale, w.dtype, threshold(p),
                                           seed, sel_bh, sel_row)
    compare_fwd(w, p, to_host(o, w.dtype), lse.cpu().numpy(), sel_bh, sel_row, o64, l64)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed,p", [(1, 0.25), (0xFFFFFFFF00000001, 0.5), (987654321, 0.04),
                                    (77, 1 / 256), (78, 255 / 256)])
def test_dropout_keep_mask_is_bit_exact(seed, p, causal, d):
    """Q = 0 and V = I: O[q, k] > 0 exactly where the oracle keeps (q, k) (and k <= q).
    Thresholds t = 1 and t = 255 are the extremes the kernels' packed keep test (byte - t
    per 16-bit lane, dropped where negative) must get right; d = 64 runs the other
    forward kernel."""
    B, H, Nq, Nk = 2, 3, 300, d
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device=DEV)
    eye = torch.eye(Nk, d, dtype=torch.bfloat16, device=DEV)
    v = eye.expand(B, H, Nk, d).contiguous()
    k = torch.randn((B, H, Nk, d), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    o, _ = fa.fa_fwd_dropout(q, k, v, p, seed, causal=causal)
    torch.cuda.synchronize()
    got = (o.float() > 0).cpu().numpy()
    t = threshold(p)
    for bh in range(B * H):
        keep = oracle.dropout_keep(seed, t, bh, Nq, Nk).astype(bool)
        if causal:
            keep &= np.tril(np.ones((Nq, Nk), dtype=bool))
        assert np.array_equal(got.reshape(B * H, Nq, d)[bh], keep), f"head {bh}"


def test_dropout_zero_probability_is_fa_fwd():
    w = inputs.custom("drop_zero", 1, 4, 384, 384, 128, "bf16", True, 77)
    q, k, v = (to_dev(a, "bf16") for a in inputs.make_qkv(w))
    o0, l0 = fa.fa_fwd(q, k, v, causal=True)
    o1, l1 = fa.fa_fwd_dropout(q, k, v, 0.0, 1234, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0, l1)


def test_dropout_seed_determines_the_result():
    w = inputs.custom("drop_det", 1, 2, 256, 256, 64, "bf16", False, 78)
    q, k, v = (to_dev(a, "bf16") for a in inputs.make_qkv(w))
    a, la = fa.fa_fwd_dropout(q, k, v, 0.3, 42)
    b, lb = fa.fa_fwd_dropout(q, k, v, 0.3, 42)
    c, lc = fa.fa_fwd_dropout(q, k, v, 0.3, 43)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert torch.equal(la, lc)  # L does not see the dropout


def test_dropout_invalid_arguments_raise():
    w = inputs.custom("drop_bad", 1, 1, 64, 64, 64, "bf16", False, 79)
    q, k, v = (to_dev(a, "bf16") for a in inputs.make_qkv(w))
    for p in (1.0, -0.01, float("nan"), 0.999):
        with pytest.raises(fa.FAError):
            fa.fa_fwd_dropout(q, k, v, p, 1)
    qf, kf, vf = q.float(), k.float(), v.float()
    with pytest.raises(fa.FAError):
        fa.fa_fwd_dropout(qf, kf, vf, 0.1, 1)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def drop_factors(w, p, seed, bh):
    """Z of head bh: keep_scale where the oracle's generator keeps (q, k), else 0."""
    keep = oracle.dropout_keep(seed, threshold(p), bh, w.Nq, w.Nk)
    return keep.astype(np.float64) * keep_scale(p)


def check_grads(w, p, seed, q, k, v, dout, bh, got, ref):
    """Element-wise bounds of tests/bwd_bounds.py with the dropout factors Z."""
    a = bwd_bounds.scales(w, q, k, v, dout, bh, z=drop_factors(w, p, seed, bh))
    for nm, g, r, s in zip(("dq", "dk", "dv"), got, ref, a):
        bwd_bounds.check(f"{nm} head {bh}", g, r, s, w.dtype, say)


BWD_SHAPES = [
    ("dbwd_128", 1, 2, 128, 128, 128, "bf16", False, 81),
    ("dbwd_ragged_causal", 2, 1, 200, 333, 64, "bf16", True, 82),
    ("dbwd_ragged_d128", 1, 2, 257, 190, 128, "f16", False, 83),
    ("dbwd_causal_d128", 1, 2, 384, 384, 128, "bf16", True, 84),
]


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("spec", BWD_SHAPES, ids=[s[0] for s in BWD_SHAPES])
def test_dropout_bwd_all_rows(spec, p):
    name, B, H, Nq, Nk, d, dt, causal, seed = spec
    w = inputs.custom(name, B, H, Nq, Nk, d, dt, causal, seed)
    say(f"[dropout bwd] {w.describe()} p={p}")
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_do(w)
    rng_seed = 0xABCDEF + seed
    tq, tk, tv, tdo = (to_dev(a, dt) for a in (q, k, v, dout))
    o, lse = fa.fa_fwd_dropout(tq, tk, tv, p, rng_seed, causal=causal, scale=w.scale)
    dq, dk, dv = fa.fa_bwd_dropout(tq, tk, tv, o, lse, tdo, p, rng_seed, causal=causal,
                                   scale=w.scale)
    torch.cuda.synchronize()
    g = [oracle.widen(to_host(t, dt), dt).reshape(B * H, -1, d) for t in (dq, dk, dv)]
    for bh in range(B * H):
        ref = oracle.bwd_head_dropout_f64(q, k, v, dout, causal, w.scale, dt, threshold(p),
                                          rng_seed, bh)
        check_grads(w, p, rng_seed, q, k, v, dout, bh, [x[bh] for x in g], ref)


def test_dropout_bwd_zero_probability_is_fa_bwd():
    w = inputs.custom("dbwd_zero", 1, 2, 256, 320, 128, "bf16", True, 85)
    q, k, v = (to_dev(a, "bf16") for a in inputs.make_qkv(w))
    dout = to_dev(inputs.make_do(w), "bf16")
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    a = fa.fa_bwd(q, k, v, o, lse, dout, causal=True)
    b = fa.fa_bwd_dropout(q, k, v, o, lse, dout, 0.0, 99, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
