"""GPU: fa_fwd_split_static (partials in the library's static device array, nothing
allocated) against fa_fwd_split with a caller workspace, through the C-ABI.

Two calls in a row on one stream, the second on a smaller problem (so the array still
holds the first call's partials where the second writes fewer), then both results
are compared bit for bit with fa_fwd_split (the same kernels) and with the fp64
oracle on sampled rows under the stated bounds.  A request beyond the array's size is
refused with FA_ERR_SCRATCH before any launch.
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

CODES = {"bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16, "f32": fa.FA_DTYPE_F32}


def static_call(w, tq, tk, tv, n_splits):
    o = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=DEV)
    need = fa.fa_fwd_split_workspace(w.B, w.H, w.Nq, w.d, n_splits)
    assert 0 < need <= fa.FA_STATIC_SCRATCH_BYTES
    st = fa.fa_fwd_split_static_raw(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), w.B, w.H, w.Nq, w.Nk, w.d, int(w.causal),
                                    w.scale, CODES[w.dtype], n_splits,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_status_str(st)
    return o, lse


def test_static_scratch_matches_workspace_path():
    big = inputs.custom("static_big", 4, 8, 256, 16384, 128, "bf16", False, seed=161)
    small = inputs.custom("static_small", 1, 4, 300, 2000, 64, "bf16", True, seed=162)
    plan = [(big, 8), (small, 4)]
    data = []
    for w, n in plan:
        say(f"[no-alloc] {w.describe()} n_splits={n}")
        q, k, v = inputs.make_qkv(w)
        data.append((w, n, (q, k, v), tuple(to_dev(a, w.dtype) for a in (q, k, v))))
    got = [static_call(w, *t, n) for w, n, _, t in data]   # two calls in a row
    torch.cuda.synchronize()
    for (w, n, (q, k, v), t), (o, lse) in zip(data, got):
        o_ref, lse_ref = fa.fa_fwd_split(*t, causal=w.causal, scale=w.scale, n_splits=n)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), w.name
        sel_bh, sel_row = inputs.sample_rows(w, min(4, w.B * w.H), min(256, w.Nq))
        o64, l64 = oracle.ref_rows_f64(q, k, v, w.causal, w.scale, w.dtype, sel_bh, sel_row)
        compare(w, to_host(o, w.dtype), lse.cpu().numpy(), sel_bh, sel_row, o64, l64)
    # the first problem again, after the smaller one: the array's stale contents of the
    # second call do not leak into the result
    w, n, _, t = data[0]
    o2, lse2 = static_call(w, *t, n)
    torch.cuda.synchronize()
    assert torch.equal(o2, got[0][0]) and torch.equal(lse2, got[0][1])


def test_static_scratch_refuses_oversized_problem():
    w = inputs.custom("static_too_big", 64, 16, 4096, 128, 128, "bf16", False, seed=163)
    assert fa.fa_fwd_split_workspace(w.B, w.H, w.Nq, w.d, 2) > fa.FA_STATIC_SCRATCH_BYTES
    t = torch.empty(16, dtype=torch.bfloat16, device=DEV)  # never touched: refused first
    st = fa.fa_fwd_split_static_raw(t.data_ptr(), t.data_ptr(), t.data_ptr(), t.data_ptr(),
                                    t.data_ptr(), w.B, w.H, w.Nq, w.Nk, w.d, 0, w.scale,
                                    fa.FA_DTYPE_BF16, 2, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_ERR_SCRATCH
