"""GPU parity over a seeded sweep of random shapes, every output row against the fp64
oracle with the stated bounds.

The shapes are drawn once from a fixed seed: batch and head counts (so that the
workgroup orders for whole and split heads per XCD both occur), query and key
lengths up to 1500 (ragged tiles, Nq != Nk, single rows), d in {64, 128}, bf16 /
fp16 / fp32, causal or not, and logit scales sigma 1 or 3.  Forward (fa_fwd), key
split (fa_fwd_split with 2 to 8 ranges), backward (fa_bwd, bf16/fp16) and dropout
(fa_fwd_dropout / fa_bwd_dropout, bf16/fp16, drop probabilities 0.1 to 0.9, the
bounds of test_dropout_gpu.py) each get their own draw.
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
from parity_util import compare, say, to_dev, to_host  # noqa: E402
from sweep_specs import BWD, DROP_BWD, DROP_FWD, FWD, SPLIT, workload  # noqa: E402
from test_bwd_gpu import check_all_rows as bwd_check_all_rows  # noqa: E402
from test_dropout_gpu import check_grads, compare_fwd, run_fwd, threshold  # noqa: E402


P_DROP = (0.1, 0.3, 0.5, 0.9)


def all_rows(w):
    return np.repeat(np.arange(w.B * w.H), w.Nq), np.tile(np.arange(w.Nq), w.B * w.H)


@pytest.mark.parametrize("spec", FWD, ids=[s[0] for s in FWD])
def test_sweep_fwd(spec):
    w = workload(spec)
    say(f"[sweep fwd] {w.describe()}")
    q, k, v = inputs.make_qkv(w)
    tq, tk, tv = (to_dev(a, w.dtype) for a in (q, k, v))
    o, lse = fa.fa_fwd(tq, tk, tv, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    sel_bh, sel_row = all_rows(w)
    o64, l64 = oracle.ref_rows_f64(q, k, v, w.causal, w.scale, w.dtype, sel_bh, sel_row)
    compare(w, to_host(o, w.dtype), lse.cpu().numpy(), sel_bh, sel_row, o64, l64)


@pytest.mark.parametrize("spec", SPLIT, ids=[s[0] for s in SPLIT])
def test_sweep_split(spec):
    w = workload(spec)
    n_splits = 2 + spec[-1] % 7
    say(f"[sweep split] {w.describe()} n_splits={n_splits}")
    q, k, v = inputs.make_qkv(w)
    tq, tk, tv = (to_dev(a, w.dtype) for a in (q, k, v))
    o, lse = fa.fa_fwd_split(tq, tk, tv, causal=w.causal, scale=w.scale, n_splits=n_splits)
    torch.cuda.synchronize()
    sel_bh, sel_row = all_rows(w)
    o64, l64 = oracle.ref_rows_f64(q, k, v, w.causal, w.scale, w.dtype, sel_bh, sel_row)
    compare(w, to_host(o, w.dtype), lse.cpu().numpy(), sel_bh, sel_row, o64, l64)


@pytest.mark.parametrize("spec", BWD, ids=[s[0] for s in BWD])
def test_sweep_bwd(spec):
    bwd_check_all_rows(workload(spec))


@pytest.mark.parametrize("spec", DROP_FWD, ids=[s[0] for s in DROP_FWD])
def test_sweep_dropout_fwd(spec):
    w = workload(spec)
    p = P_DROP[spec[-1] % 4]
    rng_seed = 0x5EED0000 + spec[-1]
    say(f"[sweep dropout fwd] {w.describe()} p={p}")
    q, k, v = inputs.make_qkv(w)
    o, lse = run_fwd(w, q, k, v, p, rng_seed)
    sel_bh, sel_row = all_rows(w)
    o64, l64 = oracle.ref_rows_dropout_f64(q, k, v, w.causal, w.scale, w.dtype, threshold(p),
                                           rng_seed, sel_bh, sel_row)
    compare_fwd(w, p, to_host(o, w.dtype), lse.cpu().numpy(), sel_bh, sel_row, o64, l64)


@pytest.mark.parametrize("spec", DROP_BWD, ids=[s[0] for s in DROP_BWD])
def test_sweep_dropout_bwd(spec):
    w = workload(spec)
    p = P_DROP[spec[-1] % 2]
    rng_seed = 0xABCDEF + spec[-1]
    say(f"[sweep dropout bwd] {w.describe()} p={p}")
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_do(w)
    tq, tk, tv, tdo = (to_dev(a, w.dtype) for a in (q, k, v, dout))
    o, lse = fa.fa_fwd_dropout(tq, tk, tv, p, rng_seed, causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.fa_bwd_dropout(tq, tk, tv, o, lse, tdo, p, rng_seed, causal=w.causal,
                                   scale=w.scale)
    torch.cuda.synchronize()
    g = [oracle.widen(to_host(t, w.dtype), w.dtype).reshape(w.B * w.H, -1, w.d)
         for t in (dq, dk, dv)]
    for bh in range(w.B * w.H):
        ref = oracle.bwd_head_dropout_f64(q, k, v, dout, w.causal, w.scale, w.dtype,
                                          threshold(p), rng_seed, bh)
        check_grads(w, p, rng_seed, q, k, v, dout, bh, [x[bh] for x in g], ref)
