"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle.

This module holds none of the attention arithmetic: it draws Gaussian values,
rounds them to the storage dtype and picks sample rows.  Both sides of a parity
check receive the same arrays from here.

Recipe (the pages draw Q, K, V with ``torch.randn`` from a fixed seed; this is
the host-side, version-pinned equivalent):

* every (tensor, b, h) slice [N, d] has its own stream:
  ``numpy.random.Generator(PCG64(SeedSequence([seed, tensor_id, b, h])))``,
  ``standard_normal((N, d), dtype=float32)`` times sigma in fp32 — so any head
  can be regenerated alone;
* the fp32 draw is rounded once to the storage dtype with round-to-nearest-even
  (bf16: on the raw bits; fp16: numpy's conversion; fp32: as drawn);
* bf16 is carried as ``uint16`` bit patterns, fp16 as ``float16``, fp32 as
  ``float32``.

The workloads below are the ones the method is measured and checked on:
shapes, dtypes, causal flags and value laws.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "do": 4}
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
    # short query block against a long key/value sequence: the shape whose grid the
    # unsplit kernel under-fills (32 workgroups), measured with the key-split path
    "short_q_long_kv": Workload("short_q_long_kv", 4, 8, 256, 16384, 128, "bf16", False,
                                seed=606),
    # the forward shape the article on hncyxsy.com times in its section 6.4 (B=8, H=16,
    # N=4096, d=64, non-causal): a large d = 64 grid, measured as context
    "pages_d64": Workload("pages_d64", 8, 16, 4096, 4096, 64, "bf16", False, seed=707),
}

# seed of the row sample drawn for the largest workloads
SAMPLE_SEED = 9001


def _bf16_bits_fast(x: np.ndarray):
    """fp64 -> bf16 nearest-even on the raw bits: keep 7 of the 52 fraction bits,
    adding half an ulp minus one plus the kept lsb (ties to even), then rebias the
    exponent from 1023 to 127.  Returns (bits, ok) where ok marks the elements whose
    result is a normal bf16 number; the others need the general path."""
    u = x.view(np.uint64)
    r = (u + np.uint64((1 << 44) - 1) + ((u >> np.uint64(45)) & np.uint64(1))) >> np.uint64(45)
    sign = (r >> np.uint64(18)) & np.uint64(1)
    e = ((r >> np.uint64(7)) & np.uint64(0x7FF)).astype(np.int64) - 1023 + 127
    frac = r & np.uint64(0x7F)
    ok = (e >= 1) & (e <= 254) & np.isfinite(x)
    bits = (sign << np.uint64(15)) | (np.clip(e, 0, 255).astype(np.uint64) << np.uint64(7)) | frac
    return bits.astype(np.uint16), ok


def round_fp64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage dtype, nearest-even, with no double rounding."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)  # a single IEEE rounding, nearest-even
    if dtype == "bf16":
        bits, ok = _bf16_bits_fast(x)
        if ok.all():
            return bits
        bits[~ok] = _round_general(x[~ok], dtype)
        return bits
    return _round_general(x, dtype)


def _round_general(x: np.ndarray, dtype: str) -> np.ndarray:
    """Scaling-based rounding that also covers zeros, subnormals, overflow and NaN."""
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
    """fp32 draw for one (tensor, b, h) slice."""
    ss = np.random.SeedSequence([int(seed), TENSOR_IDS[tensor], int(b), int(h)])
    rng = np.random.Generator(np.random.PCG64(ss))
    x = rng.standard_normal((n, d), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def round_fp32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the storage dtype, nearest-even (in place for bf16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    # bf16: add 0x7fff plus the lsb that is kept, then drop the low 16 bits; a carry
    # into the exponent is the correct rounding, and overflow lands on +-inf
    nan = np.isnan(x)
    u = x.view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    out = u.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def make_tensor(w: Workload, tensor: str) -> np.ndarray:
    """[B, H, N, d] array in the storage dtype."""
    n = w.Nq if tensor in ("q", "do") else w.Nk
    sigma = {"q": w.sigma_q, "k": w.sigma_k, "v": w.sigma_v, "do": 1.0}[tensor]
    out = np.empty((w.B, w.H, n, w.d), dtype=STORAGE[w.dtype])

    def fill(bh):
        b, h = divmod(bh, w.H)
        out[b, h] = round_fp32(head_values(w.seed, tensor, b, h, n, w.d, sigma), w.dtype)

    heads = range(w.B * w.H)
    if w.B * w.H * n * w.d < (1 << 22):
        for bh in heads:
            fill(bh)
    else:  # each head has its own stream, so heads can be drawn in parallel
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, heads))
    return out


def make_qkv(w: Workload):
    return make_tensor(w, "q"), make_tensor(w, "k"), make_tensor(w, "v")


def make_do(w: Workload) -> np.ndarray:
    """The output gradient dO for the backward pass: [B, H, Nq, d], N(0, 1) per element,
    drawn like q, k and v from its own per-head stream."""
    return make_tensor(w, "do")


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


# ---------------------------------------------------------------------------
# caller masks: seeded boolean patterns and their bit-packed form
# ---------------------------------------------------------------------------

MASK_KINDS = ("random", "key_padding", "sliding_window", "block", "empty_rows")


def pack_mask(visible: np.ndarray) -> np.ndarray:
    """Boolean [..., Nq, Nk] (True = key visible) -> uint32 words [..., Nq, ceil(Nk/32)]
    with key k in bit k % 32 of word k // 32 (bits past Nk are 0)."""
    vis = np.asarray(visible, dtype=bool)
    nk = vis.shape[-1]
    w = -(-nk // 32)
    pad = np.zeros(vis.shape[:-1] + (w * 32,), dtype=bool)
    pad[..., :nk] = vis
    bits = pad.reshape(vis.shape[:-1] + (w, 32)).astype(np.uint64)
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (bits * weights).sum(axis=-1).astype(np.uint32)


def make_mask(kind: str, mask_b: int, mask_h: int, Nq: int, Nk: int, seed: int,
              density: float = 0.5, window: int = 100, tile: int = 64) -> np.ndarray:
    """A seeded boolean mask [mask_b, mask_h, Nq, Nk] (True = visible):

    * random:         each (q, k) visible with probability `density`;
    * key_padding:    per batch a valid key count drawn in [Nk/4, Nk]; keys past it hidden
                      (the same for every head and query);
    * sliding_window: key k visible to query q iff |q - k| <= window;
    * block:          tile x tile blocks, each wholly visible with probability `density`;
    * empty_rows:     random, and about one row in eight with no visible key.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), 77])))
    shape = (mask_b, mask_h, Nq, Nk)
    if kind == "random":
        return rng.random(shape) < density
    if kind == "key_padding":
        valid = rng.integers(max(1, Nk // 4), Nk + 1, size=mask_b)
        vis = np.arange(Nk)[None, :] < valid[:, None]
        return np.broadcast_to(vis[:, None, None, :], shape).copy()
    if kind == "sliding_window":
        q = np.arange(Nq)[:, None]
        k = np.arange(Nk)[None, :]
        return np.broadcast_to(np.abs(q - k) <= window, shape).copy()
    if kind == "block":
        tb = rng.random((mask_b, mask_h, -(-Nq // tile), -(-Nk // tile))) < density
        vis = np.repeat(np.repeat(tb, tile, axis=2), tile, axis=3)
        return vis[:, :, :Nq, :Nk].copy()
    if kind == "empty_rows":
        vis = rng.random(shape) < density
        vis[rng.random(shape[:3]) < 0.125] = False
        return vis
    raise ValueError(kind)
