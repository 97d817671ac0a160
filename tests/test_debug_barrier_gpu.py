"""The full-barrier check build against the optimised library, bit for bit.

libfa_debug.so is libfa.so compiled with FA_DEBUG_FULL_BARRIER: every workgroup
barrier of every kernel first waits for all of the wave's outstanding memory
operations (global loads, DMA into LDS, LDS reads and writes), where the optimised
kernels keep loads of later tiles in flight across barriers and wait for them only
where the schedule says their buffers are first read.  Both builds do the same
arithmetic in the same order, so their outputs must agree bit for bit; a difference
would mean some kernel reads an LDS buffer or a register that a pending load has not
filled yet.  Each case runs one call through each library on the same inputs: every
forward kernel (d = 128 phase-alternating, d = 64 with and without key groups, fp32,
key splits and their merge, dropout, caller masks) and the backward kernels.
"""
import numpy as np
import pytest

from flashattention_tiling_online_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import flashattention_tiling_online_amd as fa  # noqa: E402
from flashattention_tiling_online_amd import binding  # noqa: E402
from parity_util import DEV, say, to_dev  # noqa: E402


@pytest.fixture(scope="module")
def debug_lib():
    binding.lib()  # the optimised library is loaded first
    return binding.load_library(binding.DEBUG_LIB_PATH)


def both(monkeypatch, debug_lib, call):
    """call() through libfa.so, then through libfa_debug.so; both results."""
    a = call()
    torch.cuda.synchronize()
    with monkeypatch.context() as m:
        m.setattr(binding, "_lib", debug_lib)
        b = call()
        torch.cuda.synchronize()
    return a, b


def same(a, b):
    for x, y in zip(a, b):
        if x.dtype in (torch.bfloat16, torch.float16):
            x, y = x.view(torch.int16), y.view(torch.int16)
        elif x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), "the check build differs from the optimised build"


FWD = [
    # (B, H, Nq, Nk, d, dtype, causal)
    (1, 4, 1000, 1000, 128, "bf16", True),     # d = 128 phase-alternating kernel
    (1, 3, 300, 777, 128, "f16", False),
    (2, 4, 700, 700, 64, "bf16", True),        # d = 64 key groups (small grid)
    (4, 16, 600, 600, 64, "bf16", True),       # d = 64, 128-row workgroups
    (1, 2, 300, 200, 64, "f32", False),        # fp32 kernel
]


@pytest.mark.parametrize("case", FWD, ids=[f"{c[5]}_d{c[4]}_{'c' if c[6] else 'n'}_{c[0]}x{c[1]}x{c[2]}"
                                           for c in FWD])
def test_forward_bits(monkeypatch, debug_lib, case):
    B, H, Nq, Nk, d, dt, causal = case
    w = inputs.custom("dbg_fwd", B, H, Nq, Nk, d, dt, causal, seed=Nq + Nk + d)
    q, k, v = (to_dev(a, dt) for a in inputs.make_qkv(w))
    say(f"[check build] fa_fwd {w.describe()}")
    same(*both(monkeypatch, debug_lib, lambda: fa.fa_fwd(q, k, v, causal=causal, scale=w.scale)))


@pytest.mark.parametrize("d", [128, 64])
def test_split_and_merge_bits(monkeypatch, debug_lib, d):
    w = inputs.custom("dbg_split", 2, 4, 256, 4000, d, "bf16", True, seed=d)
    q, k, v = (to_dev(a, "bf16") for a in inputs.make_qkv(w))
    same(*both(monkeypatch, debug_lib,
               lambda: fa.fa_fwd_split(q, k, v, causal=True, scale=w.scale, n_splits=5)))


@pytest.mark.parametrize("d", [128, 64])
def test_dropout_bits(monkeypatch, debug_lib, d):
    w = inputs.custom("dbg_drop", 1, 4, 500, 600, d, "bf16", True, seed=3 * d)
    q, k, v = (to_dev(a, "bf16") for a in inputs.make_qkv(w))
    dout = to_dev(inputs.make_do(w), "bf16")

    def run():
        o, lse = fa.fa_fwd_dropout(q, k, v, 0.25, 99, causal=True, scale=w.scale)
        return (o, lse) + tuple(fa.fa_bwd_dropout(q, k, v, o, lse, dout, 0.25, 99, causal=True,
                                                  scale=w.scale))
    same(*both(monkeypatch, debug_lib, run))


@pytest.mark.parametrize("d", [128, 64])
def test_masked_bits(monkeypatch, debug_lib, d):
    w = inputs.custom("dbg_mask", 1, 3, 400, 500, d, "bf16", False, seed=5 * d)
    q, k, v = (to_dev(a, "bf16") for a in inputs.make_qkv(w))
    dout = to_dev(inputs.make_do(w), "bf16")
    vis = inputs.make_mask("random", 1, 3, 400, 500, seed=d)
    mask = torch.from_numpy(inputs.pack_mask(vis).view(np.int32)).to(DEV)

    def run():
        o, lse = fa.fa_fwd_masked(q, k, v, mask, scale=w.scale)
        return (o, lse) + tuple(fa.fa_bwd_masked(q, k, v, mask, o, lse, dout, scale=w.scale))
    same(*both(monkeypatch, debug_lib, run))


@pytest.mark.parametrize("d,causal", [(128, True), (128, False), (64, True)])
def test_backward_bits(monkeypatch, debug_lib, d, causal):
    w = inputs.custom("dbg_bwd", 1, 4, 640, 520, d, "bf16", causal, seed=7 * d)
    q, k, v = (to_dev(a, "bf16") for a in inputs.make_qkv(w))
    dout = to_dev(inputs.make_do(w), "bf16")
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=w.scale)
    same(*both(monkeypatch, debug_lib,
               lambda: fa.fa_bwd(q, k, v, o, lse, dout, causal=causal, scale=w.scale)))
