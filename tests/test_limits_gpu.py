"""GPU parity at the largest offsets the forward (and the backward, last test) accepts.

fa_fwd limits a head to Nq*d < 2^31 elements (in-head offsets are 32-bit) and lets
the whole tensor exceed 2^31 (head offsets are 64-bit).  Shape: B=1, H=2,
Nq = 2^24 - 256 (Nq*d = 2^31 - 32768), Nk = 64, d = 128, bf16, both masks, so Q and O
are 8 GiB each and their last rows sit past byte 2^33.

Q is zero except for 64 seeded rows per head placed at the end of the head, at its
middle and just past 2^30 elements, all at row index >= 63 so that every key is
visible to them under either mask.  Those rows are checked against the fp64 oracle
on the small problem made of the same 64 query rows and the same K, V (a row's
output depends only on its own query row, K and V).  Zero rows have a closed form:
all scores are 0, so O is the mean of the visible value rows and L = ln(#visible);
the first 64 rows (causal: 1..64 visible keys) and a few far rows are checked
against it with the stated bounds.
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

NQ = (1 << 24) - 256
NK, D, H = 64, 128, 2
N_PLACED = 64


def placed_rows():
    """Row indices (per head) that receive the seeded query rows: 32 at the end, 16 at
    the middle and 16 just past 2^30 / d rows."""
    end = np.arange(NQ - 32, NQ)
    mid = np.arange(NQ // 2, NQ // 2 + 16)
    far = np.arange((1 << 30) // D + 5, (1 << 30) // D + 21)
    r = np.concatenate([far, mid, end]).astype(np.int64)
    assert r.size == N_PLACED and r.min() >= NK - 1 and np.unique(r).size == N_PLACED
    return r


@pytest.mark.parametrize("causal", [False, True])
def test_largest_offsets(causal):
    small = inputs.custom("limits_rows", 1, H, N_PLACED, NK, D, "bf16", False, seed=61)
    say(f"[limits] B=1 H={H} Nq={NQ} Nk={NK} d={D} bf16 causal={causal}; rows from {small.describe()}")
    q_s, k, v = inputs.make_qkv(small)
    rows = placed_rows()
    tq = torch.zeros((1, H, NQ, D), dtype=torch.bfloat16, device=DEV)
    tq_s = to_dev(q_s, "bf16")
    idx = torch.from_numpy(rows).to(DEV)
    for h in range(H):
        tq[0, h].index_copy_(0, idx, tq_s[0, h])
    tk, tv = to_dev(k, "bf16"), to_dev(v, "bf16")
    o, lse = fa.fa_fwd(tq, tk, tv, causal=causal, scale=small.scale)
    torch.cuda.synchronize()

    # the placed rows against the oracle on the small problem (all keys visible)
    o_rows = torch.stack([o[0, h].index_select(0, idx) for h in range(H)]).unsqueeze(0)
    l_rows = torch.stack([lse[0, h].index_select(0, idx) for h in range(H)]).unsqueeze(0)
    sel_bh = np.repeat(np.arange(H), N_PLACED)
    sel_row = np.tile(np.arange(N_PLACED), H)
    o64, l64 = oracle.ref_rows_f64(q_s, k, v, False, small.scale, "bf16", sel_bh, sel_row)
    compare(small, to_host(o_rows, "bf16"), l_rows.cpu().numpy(), sel_bh, sel_row, o64, l64)

    # zero query rows: O = mean of the visible value rows, L = ln(#visible)
    zero_rows = np.concatenate([np.arange(NK), [NK + 7, (1 << 23) + 3, NQ - 40]]).astype(np.int64)
    assert not np.isin(zero_rows, rows).any()
    zidx = torch.from_numpy(zero_rows).to(DEV)
    v64 = oracle.widen(v, "bf16")[0]  # [H, Nk, d]
    for h in range(H):
        oz = oracle.widen(to_host(o[0, h].index_select(0, zidx), "bf16"), "bf16")
        lz = lse[0, h].index_select(0, zidx).cpu().numpy().astype(np.float64)
        n_vis = np.minimum(zero_rows + 1, NK) if causal else np.full(zero_rows.size, NK)
        ref = np.stack([v64[h, :n].mean(axis=0) for n in n_vis])
        err = np.abs(oz - ref)
        say(f"  zero rows head {h}: max|dO|={err.max():.3e} max|dL|={np.abs(lz - np.log(n_vis)).max():.3e}")
        assert err.max() <= 1e-2 and err.mean() <= 1e-3
        assert np.abs(lz - np.log(n_vis)).max() <= 1e-3
    del tq, o, lse
    torch.cuda.empty_cache()


NK_BIG = (1 << 24) - 256


def placed_keys():
    """Key indices (per head) that receive the seeded key and value rows: 32 at the
    end, 16 at the middle and 16 just past 2^30 / d rows."""
    end = np.arange(NK_BIG - 32, NK_BIG)
    mid = np.arange(NK_BIG // 2, NK_BIG // 2 + 16)
    far = np.arange((1 << 30) // D + 5, (1 << 30) // D + 21)
    r = np.concatenate([far, mid, end]).astype(np.int64)
    assert r.size == NK and np.unique(r).size == NK
    return r


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_split_hint", "fa_fwd_split_256"])
def test_largest_key_offsets(entry):
    """Nk = 2^24 - 256 keys per head (Nk*d just under 2^31; K and V 8 GiB each), zero
    except 64 seeded key/value rows per head placed at the end, the middle and just past
    2^30 elements; 64 seeded query rows (sigma 3 for Q and K, so the placed keys carry
    most of the weight).  Exact result: the fp64 oracle on the 64 placed keys, folded
    with the (+) of the blog page with the zero keys' state (m = 0, d = Nk - 64,
    o~ = 0) by the oracle's own merge."""
    small = inputs.custom("limits_keys", 1, H, 64, NK, D, "bf16", False, seed=67,
                          sigma_q=3.0, sigma_k=3.0)
    say(f"[limits] B=1 H={H} Nq=64 Nk={NK_BIG} d={D} bf16 non-causal via {entry}; rows from {small.describe()}")
    q, k_s, v_s = inputs.make_qkv(small)
    keys = placed_keys()
    kidx = torch.from_numpy(keys).to(DEV)
    tk = torch.zeros((1, H, NK_BIG, D), dtype=torch.bfloat16, device=DEV)
    tv = torch.zeros((1, H, NK_BIG, D), dtype=torch.bfloat16, device=DEV)
    tks, tvs = to_dev(k_s, "bf16"), to_dev(v_s, "bf16")
    for h in range(H):
        tk[0, h].index_copy_(0, kidx, tks[0, h])
        tv[0, h].index_copy_(0, kidx, tvs[0, h])
    tq = to_dev(q, "bf16")
    if entry == "fa_fwd":
        o, lse = fa.fa_fwd(tq, tk, tv, causal=False, scale=small.scale)
    else:
        ns = None if entry == "fa_fwd_split_hint" else 256
        o, lse = fa.fa_fwd_split(tq, tk, tv, causal=False, scale=small.scale, n_splits=ns)
    torch.cuda.synchronize()

    sel_bh = np.repeat(np.arange(H), 64)
    sel_row = np.tile(np.arange(64), H)
    o_s, l_s = oracle.ref_rows_f64(q, k_s, v_s, False, small.scale, "bf16", sel_bh, sel_row)
    zero_state = np.concatenate([[0.0, float(NK_BIG - NK)], np.zeros(D)])
    o64 = np.empty_like(o_s)
    l64 = np.empty_like(l_s)
    for i in range(o_s.shape[0]):
        st = oracle.merge(np.concatenate([[l_s[i], 1.0], o_s[i]]), zero_state)
        o64[i] = st[2:] / st[1]  # the state carries o~ unnormalised
        l64[i] = st[0] + np.log(st[1])
    say(f"  weight of the placed keys: min {np.exp(l_s - l64).min():.3f}, median {np.median(np.exp(l_s - l64)):.3f}")
    compare(small, to_host(o, "bf16"), lse.cpu().numpy(), sel_bh, sel_row, o64, l64)
    del tk, tv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
def test_backward_largest_offsets(causal):
    """fa_bwd at Nq = 2^24 - 256 (Q, dO, O and dQ 8 GiB each), Nk = 64: Q and dO are zero
    except the 64 seeded rows per head placed as above.  A zero dO row has dP = 0 and
    D = 0, so dS = 0: it adds nothing to dK and dV and its dQ row is exactly 0.  So dK,
    dV and the placed dQ rows equal the fp64 oracle's gradients of the small problem
    made of the placed rows (all 64 keys visible to each), within the backward's
    bounds, and the other dQ rows are exactly zero."""
    import bwd_bounds  # noqa: E402
    small = inputs.custom("limits_bwd", 1, H, N_PLACED, NK, D, "bf16", False, seed=63)
    say(f"[limits bwd] B=1 H={H} Nq={NQ} Nk={NK} d={D} bf16 causal={causal}; rows from {small.describe()}")
    q_s, k, v = inputs.make_qkv(small)
    do_s = inputs.make_do(small)
    rows = placed_rows()
    idx = torch.from_numpy(rows).to(DEV)
    tq = torch.zeros((1, H, NQ, D), dtype=torch.bfloat16, device=DEV)
    tdo = torch.zeros((1, H, NQ, D), dtype=torch.bfloat16, device=DEV)
    tq_s, tdo_s = to_dev(q_s, "bf16"), to_dev(do_s, "bf16")
    for h in range(H):
        tq[0, h].index_copy_(0, idx, tq_s[0, h])
        tdo[0, h].index_copy_(0, idx, tdo_s[0, h])
    tk, tv = to_dev(k, "bf16"), to_dev(v, "bf16")
    o, lse = fa.fa_fwd(tq, tk, tv, causal=causal, scale=small.scale)
    dq, dk, dv = fa.fa_bwd(tq, tk, tv, o, lse, tdo, causal=causal, scale=small.scale)
    torch.cuda.synchronize()
    zero_rows = torch.from_numpy(np.array([0, 1, NK + 7, (1 << 23) + 3, NQ - 40], dtype=np.int64)).to(DEV)
    for h in range(H):
        ref_dq, ref_dk, ref_dv = oracle.bwd_head_f64(q_s, k, v, do_s, False, small.scale, "bf16", h)
        got_dq = oracle.widen(to_host(dq[0, h].index_select(0, idx), "bf16"), "bf16")
        got_dk = oracle.widen(to_host(dk[0, h], "bf16"), "bf16")
        got_dv = oracle.widen(to_host(dv[0, h], "bf16"), "bf16")
        say(f"  head {h}")
        a_q, a_k, a_v = bwd_bounds.scales(small, q_s, k, v, do_s, h)
        bwd_bounds.check("dq (placed rows)", got_dq, ref_dq, a_q, "bf16", say)
        bwd_bounds.check("dk", got_dk, ref_dk, a_k, "bf16", say)
        bwd_bounds.check("dv", got_dv, ref_dv, a_v, "bf16", say)
        assert bool((dq[0, h].index_select(0, zero_rows) == 0).all())
    del tq, tdo, o, lse, dq
    torch.cuda.empty_cache()
