"""The seeded random shapes of the GPU sweep (test_sweep_gpu.py), importable on the CPU.

Each spec is (name, B, H, Nq, Nk, d, dtype, causal, sigma_qk, seed): batch and head
counts, query and key lengths up to max_n (ragged tiles, Nq != Nk, single rows), d in
{64, 128}, one of the given dtypes, causal or not, and logit scale sigma 1 or 3.
"""
import numpy as np

from flashattention_tiling_online_amd import inputs


def draw(seed, n, dtypes, max_n, max_h):
    rs = np.random.RandomState(seed)
    out = []
    for i in range(n):
        B = int(rs.randint(1, 3))
        H = int(rs.choice([1, 2, 3, 4, 5, 8, 9][: max(1, max_h)]))
        Nq = int(rs.choice([1, 31, 33, 64, 127, 255, 257]) if rs.rand() < 0.3 else rs.randint(1, max_n + 1))
        Nk = int(rs.choice([1, 63, 65, 128, 200]) if rs.rand() < 0.3 else rs.randint(1, max_n + 1))
        d = int(rs.choice([64, 128]))
        dt = str(rs.choice(dtypes))
        causal = bool(rs.rand() < 0.5)
        sig = float(rs.choice([1.0, 3.0]))
        out.append((f"s{seed}_{i}", B, H, Nq, Nk, d, dt, causal, sig, 1000 * seed + i))
    return out


FWD = draw(7, 60, ["bf16", "bf16", "f16", "f32"], 1500, 7)
SPLIT = draw(8, 30, ["bf16", "f16", "f32"], 1500, 7)
BWD = draw(9, 20, ["bf16", "f16"], 600, 4)
DROP_FWD = draw(10, 20, ["bf16", "f16"], 1000, 7)
DROP_BWD = draw(11, 8, ["bf16", "f16"], 400, 4)


def workload(spec):
    name, B, H, Nq, Nk, d, dt, causal, sig, seed = spec
    return inputs.custom(name, B, H, Nq, Nk, d, dt, causal, seed, sigma_q=sig, sigma_k=sig)
