"""GPU parity of fa_fwd_masked (a caller's boolean mask on the scores) against the
fp64 oracle's part 5, through the C-ABI.

The blog page "Flash Attention" (Algorithm 2) masks the scaled scores before the
softmax; the mask here is bit-packed per query row (key k in bit k % 32 of word k // 32)
and may be shared over batch and heads.  Every row of ragged, rectangular, causal and
non-causal shapes of every dtype and head size is compared with the oracle under the
forward's stated bounds; rows with no visible key must be exactly O = 0 and L = -inf;
an all-visible mask must give fa_fwd's bits; a C4a-sized sample (B=1, H=16, N=8192,
d=128, causal, with a sliding window) is checked on seeded rows.
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
from parity_util import DEV, compare, say, to_dev, to_host  # noqa: E402


def mask_dev(words):
    return torch.from_numpy(words.view(np.int32)).to(DEV)


def run_masked(w, q, k, v, words):
    tq, tk, tv = (to_dev(a, w.dtype) for a in (q, k, v))
    o, lse = fa.fa_fwd_masked(tq, tk, tv, mask_dev(words), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return to_host(o, w.dtype), lse.cpu().numpy()


def check_masked(w, q, k, v, words, vis, sel_bh, sel_row):
    """Compare the selected rows; rows that see no key must be (0, -inf) exactly."""
    o_np, lse_np = run_masked(w, q, k, v, words)
    mb, mh = words.shape[:2]
    b, h = sel_bh // w.H, sel_bh % w.H
    rows_vis = vis[np.where(mb > 1, b, 0), np.where(mh > 1, h, 0), sel_row]
    if w.causal:
        rows_vis = rows_vis & (np.arange(w.Nk)[None, :] <= sel_row[:, None])
    live = rows_vis.any(axis=1)
    o_all = oracle.widen(o_np.reshape(-1, w.d), w.dtype)
    l_all = lse_np.reshape(-1)
    dead = (sel_bh * w.Nq + sel_row)[~live]
    assert (o_all[dead] == 0).all(), "a row with no visible key must give O = 0"
    assert np.isneginf(l_all[dead]).all(), "a row with no visible key must give L = -inf"
    if live.any():
        o64, l64 = oracle.ref_rows_masked_f64(q, k, v, words, w.causal, w.scale, w.dtype,
                                              sel_bh[live], sel_row[live])
        compare(w, o_np, lse_np, sel_bh[live], sel_row[live], o64, l64)
    return int((~live).sum())


CASES = [
    # (B, H, Nq, Nk, d, dtype, causal, kind, mask_b, mask_h, sigma_qk, density)
    (1, 2, 200, 333, 128, "bf16", False, "random", 1, 2, 1.0, 0.5),
    (2, 3, 257, 190, 64, "bf16", True, "empty_rows", 2, 3, 1.0, 0.5),
    (1, 4, 300, 1000, 128, "f16", False, "key_padding", 1, 1, 1.0, 0.5),
    (2, 2, 640, 640, 128, "bf16", True, "sliding_window", 1, 1, 3.0, 0.5),
    (1, 2, 129, 65, 64, "f32", False, "random", 1, 1, 1.0, 0.5),
    (1, 2, 190, 257, 128, "f32", True, "block", 1, 2, 1.0, 0.5),
    (1, 3, 512, 512, 64, "bf16", False, "block", 1, 3, 1.0, 0.5),
    (1, 1, 1, 1, 128, "bf16", False, "random", 1, 1, 1.0, 0.5),
    (2, 2, 33, 1500, 64, "bf16", False, "empty_rows", 2, 1, 1.0, 0.5),
    (1, 2, 1000, 1000, 128, "bf16", True, "random", 1, 2, 3.0, 0.05),
    (2, 4, 700, 900, 128, "f16", False, "empty_rows", 2, 4, 1.0, 0.3),
    (1, 2, 300, 300, 64, "f32", True, "sliding_window", 1, 1, 1.0, 0.5),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[7]}_{c[5]}_d{c[4]}_{'c' if c[6] else 'n'}_{i}"
                                             for i, c in enumerate(CASES)])
def test_masked_all_rows(case):
    B, H, Nq, Nk, d, dt, causal, kind, mb, mh, sig, dens = case
    w = inputs.custom(f"mask_{kind}", B, H, Nq, Nk, d, dt, causal, seed=500 + Nq + Nk,
                      sigma_q=sig, sigma_k=sig)
    say(f"[mask] {w.describe()} kind={kind} mask=[{mb},{mh}] density={dens}")
    q, k, v = inputs.make_qkv(w)
    vis = inputs.make_mask(kind, mb, mh, Nq, Nk, seed=Nq * 7 + Nk, density=dens, window=60,
                           tile=48)
    words = inputs.pack_mask(vis)
    sel_bh = np.repeat(np.arange(B * H), Nq)
    sel_row = np.tile(np.arange(Nq), B * H)
    n_dead = check_masked(w, q, k, v, words, vis, sel_bh, sel_row)
    say(f"  rows with no visible key: {n_dead}")


@pytest.mark.parametrize("d,dt,causal", [(128, "bf16", True), (128, "f16", False),
                                         (64, "bf16", True), (64, "f32", False),
                                         (128, "f32", True)])
def test_all_visible_mask_gives_fa_fwd_bits(d, dt, causal):
    # d = 64: a grid of more than 256 workgroups of 128 rows, where fa_fwd runs the same
    # kernel as the masked forward (smaller d = 64 grids take key groups there)
    B, H = (2, 3) if d == 128 else (4, 16)
    w = inputs.custom("mask_all", B, H, 600, 270, d, dt, causal, seed=61)
    q, k, v = inputs.make_qkv(w)
    words = inputs.pack_mask(np.ones((1, 1, w.Nq, w.Nk), bool))
    o_m, l_m = run_masked(w, q, k, v, words)
    tq, tk, tv = (to_dev(a, dt) for a in (q, k, v))
    o, lse = fa.fa_fwd(tq, tk, tv, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(o_m, to_host(o, dt)) and np.array_equal(l_m, lse.cpu().numpy())


def test_bits_past_the_last_key_are_ignored():
    w = inputs.custom("mask_tail", 1, 2, 130, 77, 128, "bf16", False, seed=62)
    q, k, v = inputs.make_qkv(w)
    vis = inputs.make_mask("random", 1, 2, 130, 77, seed=5)
    words = inputs.pack_mask(vis)
    noisy = words.copy()
    noisy[..., -1] |= np.uint32(0xFFFFFFFF) << np.uint32(77 % 32)   # keys 77..95
    a = run_masked(w, q, k, v, words)
    b = run_masked(w, q, k, v, noisy)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_masked_c4a_sample():
    """N=8192 causal, 16 heads, d=128, a sliding window of 1024 keys shared by all heads:
    4 seeded heads x 256 seeded rows against the oracle."""
    w = inputs.custom("mask_8k_window", 1, 16, 8192, 8192, 128, "bf16", True, seed=404)
    say(f"[mask] {w.describe()} sliding window 1024")
    q, k, v = inputs.make_qkv(w)
    qi = np.arange(8192)[:, None]
    kj = np.arange(8192)[None, :]
    vis = (np.abs(qi - kj) <= 1024)[None, None]
    words = inputs.pack_mask(vis)
    sel_bh, sel_row = inputs.sample_rows(w, 4, 256)
    assert check_masked(w, q, k, v, words, vis, sel_bh, sel_row) == 0


# ---------------------------------------------------------------------------
# backward with the same mask (fa_bwd_masked)
# ---------------------------------------------------------------------------

BWD_CASES = [
    # (B, H, Nq, Nk, d, dtype, causal, kind, mask_b, mask_h, density)
    (1, 2, 200, 333, 128, "bf16", False, "random", 1, 2, 0.5),
    (2, 2, 257, 190, 64, "bf16", True, "empty_rows", 2, 1, 0.5),
    (1, 3, 300, 260, 128, "f16", True, "sliding_window", 1, 1, 0.5),
    (1, 2, 129, 400, 64, "f16", False, "key_padding", 1, 1, 0.5),
    (1, 2, 384, 384, 128, "bf16", False, "block", 1, 2, 0.5),
    (2, 2, 300, 300, 128, "bf16", True, "empty_rows", 2, 2, 0.2),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[f"{c[7]}_{c[5]}_d{c[4]}_{'c' if c[6] else 'n'}_{i}"
                                                 for i, c in enumerate(BWD_CASES)])
def test_masked_backward_all_rows(case):
    import bwd_bounds
    B, H, Nq, Nk, d, dt, causal, kind, mb, mh, dens = case
    w = inputs.custom(f"mask_bwd_{kind}", B, H, Nq, Nk, d, dt, causal, seed=700 + Nq + Nk)
    say(f"[mask bwd] {w.describe()} kind={kind} mask=[{mb},{mh}] density={dens}")
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_do(w)
    vis = inputs.make_mask(kind, mb, mh, Nq, Nk, seed=Nq * 3 + Nk, density=dens, window=50,
                           tile=32)
    words = inputs.pack_mask(vis)
    tq, tk, tv, tdo = (to_dev(a, dt) for a in (q, k, v, dout))
    tm = mask_dev(words)
    o, lse = fa.fa_fwd_masked(tq, tk, tv, tm, causal=causal, scale=w.scale)
    dq, dk, dv = fa.fa_bwd_masked(tq, tk, tv, tm, o, lse, tdo, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    g = [oracle.widen(to_host(t, dt), dt).reshape(B * H, -1, d) for t in (dq, dk, dv)]
    for bh in range(B * H):
        b, h = divmod(bh, H)
        hv = vis[b if mb > 1 else 0, h if mh > 1 else 0]
        ref = oracle.bwd_head_masked_f64(q, k, v, dout, words, causal, w.scale, dt, bh)
        a = bwd_bounds.scales(w, q, k, v, dout, bh, vis=hv)
        say(f"  head {bh}")
        for nm, got, r, s in zip(("dq", "dk", "dv"), g, ref, a):
            bwd_bounds.check(nm, got[bh], r, s, dt, say)
        live = (hv & (np.tril(np.ones((Nq, Nk), bool)) if causal else hv)).any(axis=1)
        assert (g[0][bh][~live] == 0).all(), "a row with no visible key has no gradient"


def test_masked_backward_all_visible_gives_fa_bwd_bits():
    w = inputs.custom("mask_bwd_all", 1, 2, 300, 270, 128, "bf16", True, seed=71)
    q, k, v = (to_dev(a, "bf16") for a in inputs.make_qkv(w))
    dout = to_dev(inputs.make_do(w), "bf16")
    tm = mask_dev(inputs.pack_mask(np.ones((1, 1, 300, 270), bool)))
    o, lse = fa.fa_fwd(q, k, v, causal=True, scale=w.scale)
    a = fa.fa_bwd(q, k, v, o, lse, dout, causal=True, scale=w.scale)
    b = fa.fa_bwd_masked(q, k, v, tm, o, lse, dout, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
