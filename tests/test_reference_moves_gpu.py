"""GPU parity on scores built so that the running maximum of every row moves on every key
tile, on alternate tiles, or never after the first tile.

The pages' recurrence (the course page "05_flash_attention.py", flash_attention_forward;
the blog page "Flash Attention", Algorithm 1) takes a new row maximum on every tile whose
scores exceed it and rescales l and O~ by exp(m_old - m_new).  The kernels move their
reference maximum lazily (only when a key would weigh more than a fifth of its row, or
while the row sum is small) and apply the rescale of O~ one phase later; these inputs
make that path run on every tile ("rise"), on every second tile ("stairs", whose flat
tiles raise the maximum only by the noise, below the kernels' slack) or not at all
("fall"), with and without the causal mask and with a ragged last tile; the test checks
the construction with the oracle's own count of the raises the pages' recurrence makes.

Construction (seeded): the query rows share one unit direction u, q_i = a u + noise, and
key j is k_j = r(j) u + noise, so that the scores of row i grow (or fall) along the keys
by about `step` log2 units per 64-key tile: r(j) = step * t(j) / (a * scale * log2 e) with
t(j) = j / 64 (rise), 2 floor(j / 128) (stairs) or (Nk - 1 - j) / 64 (fall).  V is
N(0, 1).  Every row of every head is compared with the fp64 oracle on the same rounded
inputs, at the usual bounds.
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

B, H, NQ, NK = 1, 2, 650, 650  # 11 key tiles, the last one ragged
A = 4.0      # length of the shared query component
STEP = 10.0  # log2 units of score growth per 64-key tile
NOISE = 0.05


def ramp(kind: str, nk: int) -> np.ndarray:
    j = np.arange(nk, dtype=np.float64)
    if kind == "rise":
        return j / 64.0
    if kind == "stairs":
        return 2.0 * np.floor(j / 128.0)
    assert kind == "fall"
    return (nk - 1 - j) / 64.0


def build(kind: str, d: int, seed: int):
    rng = np.random.default_rng(seed)
    scale = 1.0 / np.sqrt(d)
    c2 = scale * np.log2(np.e)
    q = np.empty((B, H, NQ, d))
    k = np.empty((B, H, NK, d))
    for h in range(H):
        u = rng.standard_normal(d)
        u /= np.linalg.norm(u)
        q[0, h] = A * u + NOISE * rng.standard_normal((NQ, d))
        r = STEP * ramp(kind, NK) / (A * c2)
        k[0, h] = r[:, None] * u + NOISE * rng.standard_normal((NK, d))
    v = rng.standard_normal((B, H, NK, d))
    return (inputs.round_fp64(q, "bf16"), inputs.round_fp64(k, "bf16"),
            inputs.round_fp64(v, "bf16"))


CASES = [(kind, d, causal) for kind in ("rise", "stairs", "fall") for d in (128, 64)
         for causal in (False, True)]


@pytest.mark.parametrize("kind,d,causal", CASES,
                         ids=[f"{c[0]}_d{c[1]}_{'c' if c[2] else 'n'}" for c in CASES])
def test_running_max_moves(kind, d, causal):
    seed = 900 + 10 * d + (1 if causal else 0) + {"rise": 0, "stairs": 3, "fall": 6}[kind]
    w = inputs.custom(f"moves_{kind}", B, H, NQ, NK, d, "bf16", causal, seed=seed)
    say(f"[moves] {kind} d={d} causal={causal} B={B} H={H} Nq={NQ} Nk={NK} seed={seed}")
    q, k, v = build(kind, d, seed)
    o, lse = fa.fa_fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                       causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    sel_bh = np.repeat(np.arange(B * H, dtype=np.int64), NQ)
    sel_row = np.tile(np.arange(NQ, dtype=np.int64), B * H)
    o64, l64 = oracle.ref_rows_f64(q, k, v, causal, w.scale, "bf16", sel_bh, sel_row)
    # the construction does what it claims: the pages' recurrence over 64-key tiles (part 2
    # of the oracle) raises each row's maximum on every visible tile after the first
    # (rise; under the causal mask a row that sees only the first few keys of its last
    # tile may not, as the ramp gains 10/64 log2 units a key against the noise), on at
    # least every second one (stairs) or on none (fall)
    o2, l2, raised = oracle.ref_rows_f64(q, k, v, causal, w.scale, "bf16", sel_bh, sel_row,
                                         online_key_block=64)
    tiles = np.minimum(sel_row // 64 + 1, -(-NK // 64)) if causal else np.full(sel_row.size, -(-NK // 64))
    if kind == "rise":
        assert (raised >= tiles - 2).all() and (raised == tiles - 1).mean() > 0.9
    elif kind == "stairs":
        assert (raised >= (tiles - 1) // 2).all()
    else:
        assert (raised == 0).all()
    assert np.abs(o2 - o64).max() <= 1e-12 and np.abs(l2 - l64).max() <= 1e-10
    say(f"  maximum raised per row (pages' recurrence): mean {raised.mean():.2f}")
    compare(w, to_host(o, "bf16"), lse.cpu().numpy(), sel_bh, sel_row, o64, l64)
