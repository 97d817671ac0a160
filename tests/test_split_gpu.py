"""GPU parity of the split-KV forward (fa_fwd_split) and the partial-state merge
(fa_merge), called through the C-ABI, against the fp64 oracle.

* fa_fwd_split's final (O, L) meet the same bounds as fa_fwd (parity_util.compare)
  on every row of the small workloads and on ragged, rectangular, fp16, fp32 and
  large-logit shapes, and on seeded row samples of two large ones;
* the partial states it leaves in the caller's workspace are checked range by range
  against the oracle's attention over that range's visible keys, and rows with no
  visible key in a range must hold the merge identity (L = -inf, O = 0) exactly;
* fa_merge is checked against the oracle's (+) fold of the same partial states
  (oracle.merge on (m, d, o~) = (L_r, 1, O_r); the blog page "Flash Attention"
  defines (+) on these states).
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
from parity_util import DEV, TORCH_DT, compare, say, to_dev, to_host  # noqa: E402

KEY_TILE = 64


def run_split(w, q, k, v, n_splits):
    tq, tk, tv = (to_dev(a, w.dtype) for a in (q, k, v))
    need = fa.fa_fwd_split_workspace(w.B, w.H, w.Nq, w.d, n_splits)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)  # NaN-filled fp32
    o, lse = fa.fa_fwd_split(tq, tk, tv, causal=w.causal, scale=w.scale, n_splits=n_splits,
                             workspace=ws)
    torch.cuda.synchronize()
    return o, lse, ws


def plan(Nk, n_splits):
    """The key ranges the header specifies for (Nk, n_splits)."""
    nkt = -(-Nk // KEY_TILE)
    s = min(n_splits, nkt)
    t = -(-nkt // s)
    n = -(-nkt // t)
    return [(KEY_TILE * t * r, min(KEY_TILE * t * (r + 1), Nk)) for r in range(n)]


def all_rows(w):
    return (np.repeat(np.arange(w.B * w.H), w.Nq), np.tile(np.arange(w.Nq), w.B * w.H))


SPLIT_CASES = [
    # (workload or custom spec, n_splits, sampled)
    ("mh_d64", 4, False),
    ("mh_d64_causal", 4, False),
    ("single_head_fp32", 4, False),
    (("ragged_causal_d128", 1, 2, 300, 1000, 128, "bf16", True, 11), 3, False),
    (("decode_like_f16", 2, 4, 64, 4096, 128, "f16", False, 12), 8, False),
    (("more_splits_than_tiles", 1, 1, 100, 100, 64, "bf16", False, 13), 5, False),
    (("causal_nq_lt_nk", 1, 2, 200, 700, 128, "bf16", True, 14), 6, False),
    (("f32_ragged_causal", 1, 2, 130, 333, 128, "f32", True, 15), 3, False),
    (("f16_d64_causal", 2, 3, 257, 257, 64, "f16", True, 16), 2, False),
    (("large_logits", 1, 2, 512, 4096, 128, "bf16", True, 17, 3.0, 3.0), 8, False),
    ("cross_1k_8k", 2, True),
    ("self_8k_causal", 2, True),
    ("short_q_long_kv", 8, True),
]


def _workload(spec):
    if isinstance(spec, str):
        return inputs.WORKLOADS[spec]
    name, B, H, Nq, Nk, d, dt, causal, seed, *sig = spec
    sq, sk = (sig + [1.0, 1.0])[:2]
    return inputs.custom(name, B, H, Nq, Nk, d, dt, causal, seed, sigma_q=sq, sigma_k=sk)


@pytest.mark.parametrize("spec,n_splits,sampled", SPLIT_CASES,
                         ids=[(c[0] if isinstance(c[0], str) else c[0][0]) + f"-s{c[1]}"
                              for c in SPLIT_CASES])
def test_split_matches_oracle(spec, n_splits, sampled):
    w = _workload(spec)
    ranges = plan(w.Nk, n_splits)
    say(f"[split] {w.describe()} n_splits={n_splits} -> {len(ranges)} ranges")
    q, k, v = inputs.make_qkv(w)
    o, lse, _ = run_split(w, q, k, v, n_splits)
    sel_bh, sel_row = inputs.sample_rows(w, 4, 256) if sampled else all_rows(w)
    o64, l64 = oracle.ref_rows_f64(q, k, v, w.causal, w.scale, w.dtype, sel_bh, sel_row)
    compare(w, to_host(o, w.dtype), lse.cpu().numpy(), sel_bh, sel_row, o64, l64)


def _range_oracle(qh, kh, vh, causal, scale, k0, k1):
    """Oracle (O_r, L_r) of every row of one head over keys [k0, k1) (fp64 inputs);
    rows with no visible key get (0, -inf)."""
    nq, d = qh.shape
    o = np.zeros((nq, d))
    lse = np.full(nq, -np.inf)
    if not causal:
        o[:], lse[:] = oracle.attention_f64(qh, kh[k0:k1], vh[k0:k1], False, scale)
        return o, lse
    full = np.arange(nq)[np.arange(nq) >= k1 - 1]
    if full.size:
        o[full], lse[full] = oracle.attention_f64(qh, kh[k0:k1], vh[k0:k1], False, scale,
                                                  rows=full)
    for r in range(max(k0, 0), min(k1 - 1, nq)):  # rows that see part of the range
        o_r, l_r = oracle.attention_f64(qh, kh[k0:r + 1], vh[k0:r + 1], False, scale, rows=[r])
        o[r], lse[r] = o_r[0], l_r[0]
    return o, lse


@pytest.mark.parametrize("spec,n_splits", [
    (("partials_causal", 1, 2, 300, 1000, 128, "bf16", True, 21), 3),
    (("partials_noncausal", 1, 2, 96, 700, 64, "bf16", False, 22), 4),
    (("partials_f32", 1, 1, 150, 260, 64, "f32", True, 23), 3),
    (("partials_fewer_ranges", 1, 1, 64, 100, 64, "bf16", False, 24), 5),
])
def test_split_partials_match_oracle(spec, n_splits):
    w = _workload(spec)
    ranges = plan(w.Nk, n_splits)
    say(f"[split partials] {w.describe()} ranges={ranges}")
    q, k, v = inputs.make_qkv(w)
    _, _, ws = run_split(w, q, k, v, n_splits)
    rows = w.B * w.H * w.Nq
    off = -(-(n_splits * rows * w.d * 4) // 256) * 256
    wsh = ws.cpu().numpy()
    o_part = wsh[: n_splits * rows * w.d * 4].view(np.float32).reshape(n_splits, w.B * w.H, w.Nq, w.d)
    l_part = wsh[off: off + n_splits * rows * 4].view(np.float32).reshape(n_splits, w.B * w.H, w.Nq)
    qw, kw, vw = (oracle.widen(a, w.dtype).reshape(w.B * w.H, -1, w.d) for a in (q, k, v))
    tol_max = 1e-4 if w.dtype == "f32" else 1e-2
    for r, (k0, k1) in enumerate(ranges):
        for bh in range(w.B * w.H):
            o_ref, l_ref = _range_oracle(qw[bh], kw[bh], vw[bh], w.causal, w.scale, k0, k1)
            o_got = o_part[r, bh].astype(np.float64)
            l_got = l_part[r, bh].astype(np.float64)
            empty = np.isinf(l_ref)
            assert np.array_equal(np.isinf(l_got) & (l_got < 0), empty), (r, bh)
            assert (o_got[empty] == 0).all(), (r, bh)
            vis = ~empty
            if vis.any():
                err = np.abs(o_got[vis] - o_ref[vis])
                assert err.max() <= tol_max, (r, bh, err.max())
                assert np.abs(l_got[vis] - l_ref[vis]).max() <= 1e-3, (r, bh)
    # ranges beyond the number used are not written
    if len(ranges) < n_splits:
        assert np.isnan(o_part[len(ranges):]).all()


def _fold_oracle(o_parts, l_parts):
    """oracle.merge fold of the states (L_r, 1, O_r) (empty state for L_r = -inf)."""
    P, rows, d = o_parts.shape
    o = np.empty((rows, d))
    lse = np.empty(rows)
    for i in range(rows):
        st = oracle.empty_state(d)
        for r in range(P):
            part = (oracle.empty_state(d) if np.isneginf(l_parts[r, i])
                    else np.concatenate([[l_parts[r, i], 1.0], o_parts[r, i]]))
            st = oracle.merge(st, part)
        m, dd, ot = st[0], st[1], st[2:]
        if dd == 0:
            o[i], lse[i] = 0.0, -np.inf
        else:
            o[i], lse[i] = ot / dd, m + np.log(dd)
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_merge_matches_oracle_fold(d, dtype):
    P, B, H, Nq = 5, 1, 3, 37  # 111 rows: a ragged last workgroup
    g = np.random.Generator(np.random.PCG64(2024 + d))
    l_parts = (g.standard_normal((P, B, H, Nq)) * 4.0).astype(np.float32)
    l_parts[g.random((P, B, H, Nq)) < 0.2] = -np.inf
    l_parts[:, 0, 1, 5] = -np.inf                    # a row with no visible key anywhere
    o_parts = g.standard_normal((P, B, H, Nq, d)).astype(np.float32)
    say(f"[merge] P={P} rows={B * H * Nq} d={d} dtype={dtype}")
    o, lse = fa.fa_merge(torch.from_numpy(o_parts).to(DEV), torch.from_numpy(l_parts).to(DEV),
                         dtype=TORCH_DT[dtype])
    torch.cuda.synchronize()
    o_ref, l_ref = _fold_oracle(o_parts.reshape(P, -1, d).astype(np.float64),
                                l_parts.reshape(P, -1).astype(np.float64))
    o_got = o.float().cpu().numpy().reshape(-1, d).astype(np.float64)
    l_got = lse.cpu().numpy().reshape(-1).astype(np.float64)
    empty = np.isneginf(l_ref)
    assert empty.sum() >= 1
    assert np.isneginf(l_got[empty]).all() and (o_got[empty] == 0).all()
    vis = ~empty
    assert np.abs(l_got[vis] - l_ref[vis]).max() <= 1e-5 * np.maximum(1, np.abs(l_ref[vis])).max()
    rel = {"f32": 2e-6, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}[dtype]
    bound = rel * np.abs(o_ref[vis]) + 1e-6
    assert (np.abs(o_got[vis] - o_ref[vis]) <= bound).all()


def test_split_deterministic_and_close_to_unsplit():
    w = inputs.custom("det_split", 2, 4, 512, 2048, 128, "bf16", True, 31)
    q, k, v = inputs.make_qkv(w)
    o1, l1, _ = run_split(w, q, k, v, 4)
    o2, l2, _ = run_split(w, q, k, v, 4)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    tq, tk, tv = (to_dev(a, w.dtype) for a in (q, k, v))
    o0, l0 = fa.fa_fwd(tq, tk, tv, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    diff = (o0.float() - o1.float()).abs()
    assert bool((diff <= 2e-2 + 2.0 ** -7 * o0.float().abs()).all())
    assert (l0 - l1).abs().max().item() <= 1e-3


def test_split_invalid_arguments_raise():
    w = inputs.custom("bad_split", 1, 2, 128, 1024, 64, "bf16", False, 41)
    q, k, v = (to_dev(a, w.dtype) for a in inputs.make_qkv(w))
    with pytest.raises(fa.FAError):
        fa.fa_fwd_split(q, k, v, n_splits=0)
    with pytest.raises(fa.FAError):
        fa.fa_fwd_split(q, k, v, n_splits=257)
    small = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):   # the binding checks the workspace's size first
        fa.fa_fwd_split(q, k, v, n_splits=4, workspace=small)
    # and the library refuses it too, when called directly with the true size
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, 128), dtype=torch.float32, device=DEV)
    st = fa.fa_fwd_split_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             1, 2, 128, 1024, 64, 0, w.scale, fa.FA_DTYPE_BF16, 4,
                             small.data_ptr(), small.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_ERR_INVALID_ARG
    torch.cuda.synchronize()
