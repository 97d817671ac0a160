"""GPU: the C-ABI entry points under HIP graph capture and on concurrent streams.

fa_fwd, fa_fwd_split (with its merge) and fa_bwd are captured into one graph on
preallocated buffers, through the Python binding (which passes torch's current
stream, the capture stream).  None of them allocates, synchronises or clears memory
on the stream, so the graph holds kernel nodes only.  The graph is replayed several
times with eager work in between (outputs cleared, inputs rewritten in place), and
every replay must equal the eager calls bit for bit (the kernels are deterministic),
and the forward must meet the fp64 oracle's bounds.  The same calls enqueued on
three streams at once must give the bits of the serial calls (the library keeps no
state between calls).
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


def eager(tq, tk, tv, tdo, scale, n_splits, ws_split, ws_bwd):
    o, lse = fa.fa_fwd(tq, tk, tv, causal=True, scale=scale)
    o_s, lse_s = fa.fa_fwd_split(tq, tk, tv, causal=True, scale=scale, n_splits=n_splits,
                                 workspace=ws_split)
    dq, dk, dv = fa.fa_bwd(tq, tk, tv, o, lse, tdo, causal=True, scale=scale, workspace=ws_bwd)
    torch.cuda.synchronize()
    return [t.clone() for t in (o, lse, o_s, lse_s, dq, dk, dv)]


@pytest.mark.parametrize("d", [128, 64])
def test_graph_replays_match_eager(d):
    w = inputs.custom(f"graph_d{d}", 1, 4, 1000, 1000, d, "bf16", True, seed=71 + d)
    w2 = inputs.custom(f"graph_d{d}_b", 1, 4, 1000, 1000, d, "bf16", True, seed=72 + d)
    say(f"[graph] {w.describe()}; second inputs {w2.describe()}")
    q, k, v = inputs.make_qkv(w)
    q2, k2, v2 = inputs.make_qkv(w2)
    tq, tk, tv = (to_dev(a, "bf16") for a in (q, k, v))
    gen = torch.Generator(device="cpu").manual_seed(73 + d)
    tdo = torch.randn(tq.shape, generator=gen).to(torch.bfloat16).to(DEV)
    n_splits = 4
    ws_split = torch.empty(fa.fa_fwd_split_workspace(1, 4, 1000, d, n_splits), dtype=torch.uint8,
                           device=DEV)
    ws_bwd = torch.empty(max(16, fa.fa_bwd_workspace(1, 4, 1000, d)), dtype=torch.uint8,
                         device=DEV)
    ref1 = eager(tq, tk, tv, tdo, w.scale, n_splits, ws_split, ws_bwd)

    outs = [torch.empty_like(t) for t in ref1]
    o, lse, o_s, lse_s, dq, dk, dv = outs
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.fa_fwd(tq, tk, tv, causal=True, scale=w.scale, o=o, lse=lse)
        fa.fa_fwd_split(tq, tk, tv, causal=True, scale=w.scale, n_splits=n_splits, o=o_s,
                        lse=lse_s, workspace=ws_split)
        fa.fa_bwd(tq, tk, tv, o, lse, tdo, causal=True, scale=w.scale, dq=dq, dk=dk, dv=dv,
                  workspace=ws_bwd)

    names = ("o", "lse", "o_split", "lse_split", "dq", "dk", "dv")
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan") if t.dtype == torch.float32 else 7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, ref1):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
    sel_bh = np.repeat(np.arange(4), 1000)
    sel_row = np.tile(np.arange(1000), 4)
    o64, l64 = oracle.ref_rows_f64(q, k, v, True, w.scale, "bf16", sel_bh, sel_row)
    compare(w, to_host(o, "bf16"), lse.cpu().numpy(), sel_bh, sel_row, o64, l64)

    # new inputs written into the captured buffers: the replay computes on them
    for t, a in zip((tq, tk, tv), (q2, k2, v2)):
        t.copy_(to_dev(a, "bf16"))
    ref2 = eager(tq, tk, tv, tdo, w.scale, n_splits, ws_split, ws_bwd)
    for rep in range(2):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, ref2):
            assert torch.equal(a, b), f"replay {rep} on new inputs: {name} differs"
    o64, l64 = oracle.ref_rows_f64(q2, k2, v2, True, w2.scale, "bf16", sel_bh, sel_row)
    compare(w2, to_host(o, "bf16"), lse.cpu().numpy(), sel_bh, sel_row, o64, l64)
    del graph


def test_concurrent_streams_match_serial():
    """The library keeps no state: fa_fwd, fa_fwd_split and fa_bwd enqueued on three
    streams at once (each on its own outputs and workspace) give the bits of the same
    calls made one after another on one stream."""
    w = inputs.custom("streams", 2, 4, 777, 901, 128, "bf16", True, seed=91)
    say(f"[streams] {w.describe()}")
    q, k, v = (to_dev(a, "bf16") for a in inputs.make_qkv(w))
    gen = torch.Generator(device="cpu").manual_seed(92)
    do = torch.randn(q.shape, generator=gen).to(torch.bfloat16).to(DEV)
    o0, l0 = fa.fa_fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()

    def calls(stream):
        with torch.cuda.stream(stream):
            a = fa.fa_fwd(q, k, v, causal=True, scale=w.scale)
            b = fa.fa_fwd_split(q, k, v, causal=True, scale=w.scale, n_splits=3)
            c = fa.fa_bwd(q, k, v, o0, l0, do, causal=True, scale=w.scale)
        return [*a, *b, *c]

    serial = calls(torch.cuda.current_stream())
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    results = []
    for rep in range(3):
        results.append([calls(s) for s in streams])
    torch.cuda.synchronize()
    for per_rep in results:
        for outs in per_rep:
            for a, b in zip(outs, serial):
                assert torch.equal(a, b)


def test_explicit_stream_temporaries_are_not_reused_early():
    """fa_fwd_split and fa_bwd given a stream other than torch's current one, with no
    workspace: the binding allocates the workspace (and the outputs) on that stream, so
    memory that the current stream allocates and overwrites right after the calls
    return is never the workspace the kernels are still using.  Results must equal the
    serial calls bit for bit."""
    w = inputs.custom("side_stream", 2, 8, 1500, 3000, 128, "bf16", True, seed=93)
    say(f"[side stream] {w.describe()}")
    q, k, v = (to_dev(a, "bf16") for a in inputs.make_qkv(w))
    gen = torch.Generator(device="cpu").manual_seed(94)
    do = torch.randn(q.shape, generator=gen).to(torch.bfloat16).to(DEV)
    o0, l0 = fa.fa_fwd(q, k, v, causal=True, scale=w.scale)
    ref_split = fa.fa_fwd_split(q, k, v, causal=True, scale=w.scale, n_splits=4)
    ref_bwd = fa.fa_bwd(q, k, v, o0, l0, do, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    ws_bytes = max(fa.fa_fwd_split_workspace(2, 8, 1500, 128, 4), fa.fa_bwd_workspace(2, 8, 1500, 128))
    side = torch.cuda.Stream()
    for rep in range(3):
        side.wait_stream(torch.cuda.current_stream())
        got_split = fa.fa_fwd_split(q, k, v, causal=True, scale=w.scale, n_splits=4, stream=side)
        got_bwd = fa.fa_bwd(q, k, v, o0, l0, do, causal=True, scale=w.scale, stream=side)
        # the current stream grabs and scribbles over freshly freed memory at once
        junk = [torch.full((ws_bytes // 4 + 1,), float("nan"), device=DEV) for _ in range(4)]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        del junk
        for a, b in zip((*got_split, *got_bwd), (*ref_split, *ref_bwd)):
            assert torch.equal(a, b), f"repeat {rep}: result differs from the serial call"
