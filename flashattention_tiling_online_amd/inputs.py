"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle.

This module holds none of the attention arithmetic: it draws Gaussian values,
rounds them to the storage dtype and picks sample rows.  Both sides of a parity
check receive the same arrays from here.

Recipe (the pages draw Q, K, V with ``torch.randn`` from a fixed seed; this is
the host-side, version-pinned equivalent):

* every (tensor, b, h) slice [N, d] has its own stream:
  ``numpy.random.Generator(PCG64(SeedSequence([seed, tensor_id, b, h])))``,
  ``standard_normal((N, d))`` in fp64, times sigma — so any head can be
  regenerated alone;
* the fp64 draw is rounded to the storage dtype with round-to-nearest-even,
  directly from fp64 (no double rounding through fp32);
* bf16 is carried as ``uint16`` bit patterns, fp16 as ``float16``, fp32 as
  ``float32``.

The workloads below are the ones the method is measured and checked on:
shapes, dtypes, causal flags and value laws.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

TENSOR_IDS = {"q": 1, "k": 2, "v": 3}
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    sigma_q: float = 1.0
    sigma_k: float = 1.0
    sigma_v: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        """1/sqrt(d) as the fp32 value handed to the kernel and the oracle."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> float:
        """Counted work: 4*B*H*Nq*Nk*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return f / 2 if self.causal else f

    def describe(self) -> str:
        c = "causal" if self.causal else "non-causal"
        return (f"{self.name}: B={self.B} H={self.H} Nq={self.Nq} Nk={self.Nk} d={self.d} "
                f"{self.dtype} {c}")


# Workloads: single-head fp32; batched multi-head d=64 (both masks); long sequence
# N=4096; N=8192 causal self-attention and Nq=1024/Nk=8192 cross-attention; and a
# 32K causal context whose Q and K have sigma 3 (logits of std ~9 that keep raising
# the running maximum along a row).
WORKLOADS = {
    "single_head_fp32": Workload("single_head_fp32", 1, 1, 256, 256, 64, "f32", False, seed=101),
    "mh_d64": Workload("mh_d64", 2, 8, 1024, 1024, 64, "bf16", False, seed=202),
    "mh_d64_causal": Workload("mh_d64_causal", 2, 8, 1024, 1024, 64, "bf16", True, seed=203),
    "long_4k": Workload("long_4k", 2, 8, 4096, 4096, 128, "bf16", False, seed=303),
    "self_8k_causal": Workload("self_8k_causal", 1, 16, 8192, 8192, 128, "bf16", True, seed=404),
    "cross_1k_8k": Workload("cross_1k_8k", 4, 16, 1024, 8192, 128, "bf16", False, seed=405),
    "ctx_32k_causal": Workload("ctx_32k_causal", 1, 32, 32768, 32768, 128, "bf16", True,
                               sigma_q=3.0, sigma_k=3.0, sigma_v=1.0, seed=505),
}

# seed of the row sample drawn for the largest workloads
SAMPLE_SEED = 9001


def round_fp64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage dtype, nearest-even, with no double rounding."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)  # a single IEEE rounding, nearest-even
    if dtype == "f16":
        p, emin, emax = 11, -14, 15
    elif dtype == "bf16":
        p, emin, emax = 8, -126, 127
    else:
        raise ValueError(dtype)
    _, e = np.frexp(x)
    ex = np.maximum(e.astype(np.int64) - 1, emin)
    quantum = np.ldexp(1.0, (ex - p + 1).astype(np.int32))
    with np.errstate(invalid="ignore"):
        r = np.rint(x / quantum) * quantum
    r = np.where((x == 0) | ~np.isfinite(x), x, r)
    maxfin = math.ldexp(2.0 - math.ldexp(1.0, 1 - p), emax)
    r = np.where(np.abs(r) > maxfin, np.copysign(np.inf, x), r)
    if dtype == "f16":
        return r.astype(np.float16)  # exact: r is a binary16 value
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)


def head_values(seed: int, tensor: str, b: int, h: int, n: int, d: int,
                sigma: float) -> np.ndarray:
    """fp64 draw for one (tensor, b, h) slice."""
    ss = np.random.SeedSequence([int(seed), TENSOR_IDS[tensor], int(b), int(h)])
    rng = np.random.Generator(np.random.PCG64(ss))
    return rng.standard_normal((n, d)) * sigma


def make_tensor(w: Workload, tensor: str) -> np.ndarray:
    """[B, H, N, d] array in the storage dtype."""
    n = w.Nq if tensor == "q" else w.Nk
    sigma = {"q": w.sigma_q, "k": w.sigma_k, "v": w.sigma_v}[tensor]
    out = np.empty((w.B, w.H, n, w.d), dtype=STORAGE[w.dtype])
    for b in range(w.B):
        for h in range(w.H):
            out[b, h] = round_fp64(head_values(w.seed, tensor, b, h, n, w.d, sigma), w.dtype)
    return out


def make_qkv(w: Workload):
    return make_tensor(w, "q"), make_tensor(w, "k"), make_tensor(w, "v")


def sample_rows(w: Workload, n_heads: int, n_rows: int, seed: int = SAMPLE_SEED):
    """Seeded sample of (b*H+h, row) pairs: n_heads distinct heads, n_rows distinct rows
    each (all rows when n_rows >= Nq), sorted by head then row."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, w.seed])))
    nbh = w.B * w.H
    heads = np.sort(rng.choice(nbh, size=min(n_heads, nbh), replace=False))
    bh, rows = [], []
    for hd in heads:
        if n_rows >= w.Nq:
            r = np.arange(w.Nq)
        else:
            r = np.sort(rng.choice(w.Nq, size=n_rows, replace=False))
        bh.append(np.full(r.size, hd, dtype=np.int64))
        rows.append(r.astype(np.int64))
    return np.concatenate(bh), np.concatenate(rows)


def custom(name: str, B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, causal: bool,
           seed: int, sigma_q: float = 1.0, sigma_k: float = 1.0,
           sigma_v: float = 1.0) -> Workload:
    return Workload(name, B, H, Nq, Nk, d, dtype, causal, sigma_q, sigma_k, sigma_v, seed)
