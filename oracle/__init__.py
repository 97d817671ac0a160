"""fp64 CPU oracle for the fused attention forward pass — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and the two share no code: the oracle widens the stored bf16 / fp16 /
fp32 inputs to fp64 itself and does every step of the arithmetic in
``fa_oracle.c`` (parts 1 and 2) or in :mod:`oracle.tiled` (the pages' two loop
orders, used for brute force on tiny inputs).

What is computed, and where it comes from (pages named by title / address):

* part 1, ``attention_f64`` / ``ref_rows_f64``: standard three-step attention —
  "05_flash_attention.py" course file, ``standard_attention``; scale tau and the
  mask from the "Flash Attention" blog page, Algorithm 2.
* part 2, ``online_f64`` / ``ref_online_f64``: the scalar online (m, d, o~)
  accumulator and the (+) merge — blog page, "Online Softmax" and the
  parallelisation section.
* part 3, ``attention_bwd_f64`` / ``bwd_*``: the gradients of sum(dO o O) — course
  file ``flash_attention_backward``; blog page, Algorithm 4 and the softmax-Jacobian
  derivation that follows it.
* part 4, ``philox4x32_10`` / ``*_dropout_*``: dropout on P (blog page, Algorithms 2
  and 4) with Philox4x32-10 random numbers (Salmon et al., SC'11), the reading taken
  for the generator the pages leave open.
* part 5, ``*_masked_*``: a caller's boolean mask on the scores (blog page,
  Algorithm 2, S_masked = mask(S), and Algorithm 4), bit-packed per query row; a
  row with no visible key gives O = 0 and L = -inf.
* ``softmax_online``: the one-dimensional online softmax with a per-block trace —
  course file ``online_softmax_stats``; the worked example of
  "手写 Flash Attention" (bjdmk.com.cn) section 2.2 is pinned against it.

Every function here is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, algebraic laws, brute force and an independent
library implementation; see those tests for which pin covers which function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libfa_oracle.so")

F32, F16, BF16 = 0, 1, 2
DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16}

# IEEE semantics: no fast-math, no FMA contraction, no vectorised reassociation.
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
          "-ffp-contract=off", "-fno-fast-math"]


def build(out_path: str = _LIB_PATH, src: str = _SRC, extra_flags=()) -> str:
    """Compile the oracle's C source into a shared library with gcc."""
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", out_path, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


_i64 = ctypes.c_int64
_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p
_u32p = ctypes.POINTER(ctypes.c_uint32)


def load(path: str = _LIB_PATH) -> ctypes.CDLL:
    """Load (building first if absent) an oracle library and declare its signatures."""
    if not os.path.exists(path):
        build(path)
    lib = ctypes.CDLL(path)
    lib.fa_oracle_softmax_online.argtypes = [_dp, _i64, _i64, _dp, _dp, _dp, _dp, _dp]
    lib.fa_oracle_merge.argtypes = [_i64, _dp, _dp, _dp]
    lib.fa_oracle_attention_f64.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64, ctypes.c_int,
                                            ctypes.c_double, _i64, _lp, _dp, _dp]
    lib.fa_oracle_online_f64.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64, ctypes.c_int,
                                         ctypes.c_double, _i64, _i64, _lp, _dp, _dp, _lp]
    lib.fa_ref_rows_f64.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                    ctypes.c_float, ctypes.c_int, _i64, _lp, _lp, _dp, _dp]
    lib.fa_ref_online_f64.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                      ctypes.c_float, ctypes.c_int, _i64, _lp, _lp, _i64, _dp,
                                      _dp, _lp]
    lib.fa_fwd_ref.argtypes = [_vp, _vp, _vp, _vp, ctypes.POINTER(ctypes.c_float), _i64, _i64,
                               _i64, _i64, _i64, ctypes.c_int, ctypes.c_float, ctypes.c_int]
    lib.fa_oracle_round.argtypes = [_dp, _i64, ctypes.c_int, _vp]
    raw4 = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_float,
            ctypes.c_int]
    lib.fa_oracle_attention_bwd_f64.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64,
                                                ctypes.c_int, ctypes.c_double, _dp, _dp, _dp]
    lib.fa_ref_bwd_head_f64.argtypes = raw4 + [_i64, _dp, _dp, _dp]
    lib.fa_ref_bwd_dq_rows_f64.argtypes = raw4 + [_i64, _lp, _lp, _dp]
    lib.fa_ref_bwd_rowstats_f64.argtypes = raw4 + [_i64, _lp, _lp, _dp, _dp]
    lib.fa_ref_bwd_dkv_keys_f64.argtypes = raw4 + [_dp, _dp, _i64, _lp, _lp, _dp, _dp]
    lib.fa_bwd_ref.argtypes = [_vp] * 7 + [_i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                           ctypes.c_float, ctypes.c_int]
    u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.fa_oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
    lib.fa_oracle_dropout_keep.argtypes = [ctypes.c_uint64, ctypes.c_int, _i64, _i64, _i64, _vp]
    lib.fa_oracle_attention_dropout_f64.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64, ctypes.c_int,
                                                    ctypes.c_double, ctypes.c_int,
                                                    ctypes.c_uint64, _i64, _i64, _lp, _dp, _dp]
    lib.fa_oracle_attention_bwd_dropout_f64.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64,
                                                        ctypes.c_int, ctypes.c_double,
                                                        ctypes.c_int, ctypes.c_uint64, _i64,
                                                        _dp, _dp, _dp]
    lib.fa_ref_rows_dropout_f64.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                            ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_uint64, _i64, _lp, _lp, _dp,
                                            _dp]
    lib.fa_ref_bwd_head_dropout_f64.argtypes = raw4 + [ctypes.c_int, ctypes.c_uint64, _i64, _dp,
                                                       _dp, _dp]
    lib.fa_oracle_attention_masked_f64.argtypes = [_dp, _dp, _dp, u32p, _i64, _i64, _i64,
                                                   ctypes.c_int, ctypes.c_double, _i64, _lp, _dp,
                                                   _dp]
    lib.fa_oracle_online_masked_f64.argtypes = [_dp, _dp, _dp, u32p, _i64, _i64, _i64,
                                                ctypes.c_int, ctypes.c_double, _i64, _i64, _lp,
                                                _dp, _dp]
    lib.fa_oracle_attention_bwd_masked_f64.argtypes = [_dp, _dp, _dp, _dp, u32p, _i64, _i64,
                                                       _i64, ctypes.c_int, ctypes.c_double, _dp,
                                                       _dp, _dp]
    rawm = [_vp, _vp, _vp, u32p, _i64, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
            ctypes.c_float, ctypes.c_int]
    lib.fa_ref_rows_masked_f64.argtypes = rawm + [_i64, _lp, _lp, _dp, _dp]
    lib.fa_ref_online_masked_f64.argtypes = rawm + [_i64, _lp, _lp, _i64, _dp, _dp]
    lib.fa_ref_bwd_head_masked_f64.argtypes = [_vp, _vp, _vp, _vp, u32p, _i64, _i64, _i64, _i64,
                                               _i64, _i64, _i64, ctypes.c_int, ctypes.c_float,
                                               ctypes.c_int, _i64, _dp, _dp, _dp]
    for name in ("fa_oracle_attention_masked_f64", "fa_oracle_online_masked_f64",
                 "fa_oracle_attention_bwd_masked_f64", "fa_ref_rows_masked_f64",
                 "fa_ref_online_masked_f64", "fa_ref_bwd_head_masked_f64"):
        getattr(lib, name).restype = ctypes.c_int
    for name in ("fa_oracle_philox4x32_10", "fa_oracle_dropout_keep",
                 "fa_oracle_attention_dropout_f64", "fa_oracle_attention_bwd_dropout_f64",
                 "fa_ref_rows_dropout_f64", "fa_ref_bwd_head_dropout_f64"):
        getattr(lib, name).restype = ctypes.c_int
    for name in ("fa_oracle_softmax_online", "fa_oracle_merge", "fa_oracle_attention_f64",
                 "fa_oracle_online_f64", "fa_ref_rows_f64", "fa_ref_online_f64", "fa_fwd_ref",
                 "fa_oracle_round", "fa_oracle_attention_bwd_f64", "fa_ref_bwd_head_f64",
                 "fa_ref_bwd_dq_rows_f64", "fa_ref_bwd_rowstats_f64", "fa_ref_bwd_dkv_keys_f64",
                 "fa_bwd_ref"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray, t=_dp):
    return a.ctypes.data_as(t)


# ---------------------------------------------------------------------------
# one-dimensional pieces
# ---------------------------------------------------------------------------

def softmax_online(x, block: int, L: ctypes.CDLL | None = None):
    """Online softmax of a vector read in blocks; returns (y, trace dict)."""
    L = L or lib()
    x = _f64(x)
    n = x.size
    nb = -(-n // block)
    y = np.empty(n)
    tr = {k: np.empty(nb) for k in ("run_m", "run_l", "carried", "fresh")}
    _check(L.fa_oracle_softmax_online(_ptr(x), n, block, _ptr(y), _ptr(tr["run_m"]),
                                      _ptr(tr["run_l"]), _ptr(tr["carried"]),
                                      _ptr(tr["fresh"])), "fa_oracle_softmax_online")
    return y, tr


def merge(a, b, L: ctypes.CDLL | None = None) -> np.ndarray:
    """(+) of two packed states [m, d, o~...]."""
    L = L or lib()
    a, b = _f64(a), _f64(b)
    assert a.shape == b.shape and a.ndim == 1 and a.size >= 2
    out = np.empty_like(a)
    _check(L.fa_oracle_merge(a.size - 2, _ptr(a), _ptr(b), _ptr(out)), "fa_oracle_merge")
    return out


def leaf_state(x: float, v) -> np.ndarray:
    """The state of a single visible key: (x, 1, v) — blog page, leaves of the (+) fold."""
    v = _f64(v)
    return np.concatenate([[x, 1.0], v])


def empty_state(dim: int) -> np.ndarray:
    return np.concatenate([[-np.inf, 0.0], np.zeros(dim)])


# ---------------------------------------------------------------------------
# one head, fp64 inputs
# ---------------------------------------------------------------------------

def attention_f64(q, k, v, causal: bool, scale: float, rows=None, L=None):
    """Part 1 (three-step) on one head of fp64 inputs; returns (o [n, d], lse [n])."""
    L = L or lib()
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, d = q.shape
    nk = k.shape[0]
    rows = np.arange(nq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    o = np.empty((rows.size, d))
    lse = np.empty(rows.size)
    _check(L.fa_oracle_attention_f64(_ptr(q), _ptr(k), _ptr(v), nq, nk, d, int(causal),
                                     float(scale), rows.size, _ptr(rows, _lp), _ptr(o),
                                     _ptr(lse)), "fa_oracle_attention_f64")
    return o, lse


def online_f64(q, k, v, causal: bool, scale: float, key_block: int = 0, rows=None, L=None):
    """Part 2 (scalar online accumulator); returns (o, lse, max_raised)."""
    L = L or lib()
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, d = q.shape
    nk = k.shape[0]
    rows = np.arange(nq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    o = np.empty((rows.size, d))
    lse = np.empty(rows.size)
    raised = np.empty(rows.size, dtype=np.int64)
    _check(L.fa_oracle_online_f64(_ptr(q), _ptr(k), _ptr(v), nq, nk, d, int(causal),
                                  float(scale), int(key_block), rows.size, _ptr(rows, _lp),
                                  _ptr(o), _ptr(lse), _ptr(raised, _lp)), "fa_oracle_online_f64")
    return o, lse, raised


# ---------------------------------------------------------------------------
# raw buffers ([B,H,N,d] arrays of the stored dtype), selected rows, threaded
# ---------------------------------------------------------------------------

def _raw(a: np.ndarray, dtype: str) -> np.ndarray:
    want = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    if a.dtype != want:
        raise TypeError(f"expected {want} storage for {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _split(n: int, parts: int):
    parts = max(1, min(parts, n))
    step = -(-n // parts)
    return [(i, min(i + step, n)) for i in range(0, n, step)]


def ref_rows_f64(q, k, v, causal: bool, scale: float, dtype: str, sel_bh, sel_row,
                 threads: int | None = None, online_key_block: int | None = None, L=None):
    """Oracle on selected rows of raw [B,H,N,d] buffers.

    Runs part 1 (or part 2 when ``online_key_block`` is not None) over the rows
    (sel_bh[i], sel_row[i]); the rows are split into contiguous chunks handled by
    ``threads`` host threads (ctypes releases the GIL during each call).
    Returns (o64 [n_sel, d], lse64 [n_sel]).
    """
    L = L or lib()
    q, k, v = _raw(q, dtype), _raw(k, dtype), _raw(v, dtype)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    sel_bh = np.ascontiguousarray(sel_bh, np.int64)
    sel_row = np.ascontiguousarray(sel_row, np.int64)
    n = sel_bh.size
    o = np.empty((n, d))
    lse = np.empty(n)
    raised = np.empty(n, dtype=np.int64)
    threads = threads or os.cpu_count() or 1
    code = DTYPE_CODES[dtype]

    def work(span):
        a, b = span
        if b <= a:
            return 0
        bh, rw = sel_bh[a:b], sel_row[a:b]
        if online_key_block is None:
            return L.fa_ref_rows_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Nq, Nk,
                                     d, int(causal), float(scale), code, b - a, _ptr(bh, _lp),
                                     _ptr(rw, _lp), _ptr(o[a:b]), _ptr(lse[a:b]))
        return L.fa_ref_online_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Nq, Nk, d,
                                   int(causal), float(scale), code, b - a, _ptr(bh, _lp),
                                   _ptr(rw, _lp), int(online_key_block), _ptr(o[a:b]),
                                   _ptr(lse[a:b]), _ptr(raised[a:b], _lp))

    spans = _split(n, threads)
    if len(spans) == 1:
        rcs = [work(spans[0])]
    else:
        with ThreadPoolExecutor(max_workers=len(spans)) as ex:
            rcs = list(ex.map(work, spans))
    for rc in rcs:
        _check(rc, "fa_ref_rows_f64" if online_key_block is None else "fa_ref_online_f64")
    if online_key_block is None:
        return o, lse
    return o, lse, raised


# ---------------------------------------------------------------------------
# caller masks (part 5): bit-packed rows, key k in bit k % 32 of word k // 32
# ---------------------------------------------------------------------------

def _mask_words(mask) -> np.ndarray:
    m = np.ascontiguousarray(mask)
    if m.dtype != np.uint32:
        raise TypeError("mask words must be uint32")
    return m


def attention_masked_f64(q, k, v, mask_rows, causal: bool, scale: float, rows=None, L=None):
    """Part 1 with a caller mask on one head: mask_rows [nq, ceil(nk/32)] uint32 words.
    A row with no visible key gives O = 0 and L = -inf."""
    L = L or lib()
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, d = q.shape
    nk = k.shape[0]
    m = _mask_words(mask_rows)
    assert m.shape == (nq, -(-nk // 32))
    rows = np.arange(nq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    o = np.empty((rows.size, d))
    lse = np.empty(rows.size)
    _check(L.fa_oracle_attention_masked_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(m, _u32p), nq, nk,
                                            d, int(causal), float(scale), rows.size,
                                            _ptr(rows, _lp), _ptr(o), _ptr(lse)),
           "fa_oracle_attention_masked_f64")
    return o, lse


def online_masked_f64(q, k, v, mask_rows, causal: bool, scale: float, key_block: int = 0,
                      rows=None, L=None):
    """Part 2 with a caller mask on one head; returns (o, lse)."""
    L = L or lib()
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, d = q.shape
    nk = k.shape[0]
    m = _mask_words(mask_rows)
    assert m.shape == (nq, -(-nk // 32))
    rows = np.arange(nq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    o = np.empty((rows.size, d))
    lse = np.empty(rows.size)
    _check(L.fa_oracle_online_masked_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(m, _u32p), nq, nk, d,
                                         int(causal), float(scale), int(key_block), rows.size,
                                         _ptr(rows, _lp), _ptr(o), _ptr(lse)),
           "fa_oracle_online_masked_f64")
    return o, lse


def attention_bwd_masked_f64(q, k, v, dout, mask_rows, causal: bool, scale: float, L=None):
    """Part 3 with a caller mask on one head; returns (dq, dk, dv)."""
    L = L or lib()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    nq, d = q.shape
    nk = k.shape[0]
    m = _mask_words(mask_rows)
    assert m.shape == (nq, -(-nk // 32))
    dq, dk, dv = np.empty((nq, d)), np.empty((nk, d)), np.empty((nk, d))
    _check(L.fa_oracle_attention_bwd_masked_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                                _ptr(m, _u32p), nq, nk, d, int(causal),
                                                float(scale), _ptr(dq), _ptr(dk), _ptr(dv)),
           "fa_oracle_attention_bwd_masked_f64")
    return dq, dk, dv


def ref_rows_masked_f64(q, k, v, mask, causal: bool, scale: float, dtype: str, sel_bh, sel_row,
                        threads: int | None = None, online_key_block: int | None = None, L=None):
    """ref_rows_f64 with a caller mask [mask_b, mask_h, Nq, ceil(Nk/32)] uint32 words
    (mask_b in {1, B}, mask_h in {1, H}); part 2 when online_key_block is given.
    Returns (o64 [n_sel, d], lse64 [n_sel])."""
    L = L or lib()
    q, k, v = _raw(q, dtype), _raw(k, dtype), _raw(v, dtype)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    m = _mask_words(mask)
    mb, mh = m.shape[0], m.shape[1]
    assert m.shape[2:] == (Nq, -(-Nk // 32))
    sel_bh = np.ascontiguousarray(sel_bh, np.int64)
    sel_row = np.ascontiguousarray(sel_row, np.int64)
    n = sel_bh.size
    o = np.empty((n, d))
    lse = np.empty(n)
    code = DTYPE_CODES[dtype]

    def work(span):
        a, b = span
        if b <= a:
            return 0
        bh, rw = sel_bh[a:b], sel_row[a:b]
        if online_key_block is None:
            return L.fa_ref_rows_masked_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                            _ptr(m, _u32p), mb, mh, B, H, Nq, Nk, d, int(causal),
                                            float(scale), code, b - a, _ptr(bh, _lp),
                                            _ptr(rw, _lp), _ptr(o[a:b]), _ptr(lse[a:b]))
        return L.fa_ref_online_masked_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                          _ptr(m, _u32p), mb, mh, B, H, Nq, Nk, d, int(causal),
                                          float(scale), code, b - a, _ptr(bh, _lp),
                                          _ptr(rw, _lp), int(online_key_block), _ptr(o[a:b]),
                                          _ptr(lse[a:b]))

    for rc in _threaded(n, threads, work):
        _check(rc, "fa_ref_rows_masked_f64")
    return o, lse


def bwd_head_masked_f64(q, k, v, dout, mask, causal: bool, scale: float, dtype: str, bh: int,
                        L=None):
    """Part 3 with a caller mask on head bh of raw buffers; returns fp64 (dq, dk, dv)."""
    L = L or lib()
    q, k, v, dout, B, H, Nq, Nk, d = _raw4(q, k, v, dout, dtype)
    m = _mask_words(mask)
    assert m.shape[2:] == (Nq, -(-Nk // 32))
    dq, dk, dv = np.empty((Nq, d)), np.empty((Nk, d)), np.empty((Nk, d))
    _check(L.fa_ref_bwd_head_masked_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                        dout.ctypes.data, _ptr(m, _u32p), m.shape[0], m.shape[1],
                                        B, H, Nq, Nk, d, int(causal), float(scale),
                                        DTYPE_CODES[dtype], int(bh), _ptr(dq), _ptr(dk),
                                        _ptr(dv)), "fa_ref_bwd_head_masked_f64")
    return dq, dk, dv


# ---------------------------------------------------------------------------
# gradients (part 3)
# ---------------------------------------------------------------------------

def attention_bwd_f64(q, k, v, dout, causal: bool, scale: float, L=None):
    """Part 3 on one head of fp64 inputs; returns (dq [nq, d], dk [nk, d], dv [nk, d])."""
    L = L or lib()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    nq, d = q.shape
    nk = k.shape[0]
    dq, dk, dv = np.empty((nq, d)), np.empty((nk, d)), np.empty((nk, d))
    _check(L.fa_oracle_attention_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), nq, nk, d,
                                         int(causal), float(scale), _ptr(dq), _ptr(dk),
                                         _ptr(dv)), "fa_oracle_attention_bwd_f64")
    return dq, dk, dv


def _raw4(q, k, v, dout, dtype):
    q, k, v, dout = (_raw(a, dtype) for a in (q, k, v, dout))
    B, H, Nq, d = q.shape
    return q, k, v, dout, B, H, Nq, k.shape[2], d


def bwd_head_f64(q, k, v, dout, causal: bool, scale: float, dtype: str, bh: int, L=None):
    """Part 3 on head bh of raw [B,H,N,d] buffers; returns fp64 (dq, dk, dv)."""
    L = L or lib()
    q, k, v, dout, B, H, Nq, Nk, d = _raw4(q, k, v, dout, dtype)
    dq, dk, dv = np.empty((Nq, d)), np.empty((Nk, d)), np.empty((Nk, d))
    _check(L.fa_ref_bwd_head_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                 B, H, Nq, Nk, d, int(causal), float(scale), DTYPE_CODES[dtype],
                                 int(bh), _ptr(dq), _ptr(dk), _ptr(dv)), "fa_ref_bwd_head_f64")
    return dq, dk, dv


def _threaded(n, threads, work):
    spans = _split(n, threads or os.cpu_count() or 1)
    if len(spans) <= 1:
        rcs = [work(spans[0])] if spans else []
    else:
        with ThreadPoolExecutor(max_workers=len(spans)) as ex:
            rcs = list(ex.map(work, spans))
    return rcs


def bwd_dq_rows_f64(q, k, v, dout, causal: bool, scale: float, dtype: str, sel_bh, sel_row,
                    threads: int | None = None, L=None):
    """dQ of the selected rows (part 3), threaded over the rows; returns [n_sel, d]."""
    L = L or lib()
    q, k, v, dout, B, H, Nq, Nk, d = _raw4(q, k, v, dout, dtype)
    sel_bh = np.ascontiguousarray(sel_bh, np.int64)
    sel_row = np.ascontiguousarray(sel_row, np.int64)
    dq = np.empty((sel_bh.size, d))

    def work(span):
        a, b = span
        if b <= a:
            return 0
        return L.fa_ref_bwd_dq_rows_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                        dout.ctypes.data, B, H, Nq, Nk, d, int(causal),
                                        float(scale), DTYPE_CODES[dtype], b - a,
                                        _ptr(sel_bh[a:b], _lp), _ptr(sel_row[a:b], _lp),
                                        _ptr(dq[a:b]))

    for rc in _threaded(sel_bh.size, threads, work):
        _check(rc, "fa_ref_bwd_dq_rows_f64")
    return dq


def bwd_dkv_keys_f64(q, k, v, dout, causal: bool, scale: float, dtype: str, sel_bh, sel_key,
                     threads: int | None = None, L=None):
    """dK and dV of the selected keys (part 3): the row statistics of every row of the
    heads involved first (threaded over rows), then the keys (threaded)."""
    L = L or lib()
    q, k, v, dout, B, H, Nq, Nk, d = _raw4(q, k, v, dout, dtype)
    sel_bh = np.ascontiguousarray(sel_bh, np.int64)
    sel_key = np.ascontiguousarray(sel_key, np.int64)
    heads = np.unique(sel_bh)
    lse_all = np.full(B * H * Nq, np.nan)
    D_all = np.full(B * H * Nq, np.nan)
    rb = np.repeat(heads, Nq)
    rr = np.tile(np.arange(Nq, dtype=np.int64), heads.size)
    lse_sel, D_sel = np.empty(rb.size), np.empty(rb.size)

    def stats(span):
        a, b = span
        if b <= a:
            return 0
        return L.fa_ref_bwd_rowstats_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                         dout.ctypes.data, B, H, Nq, Nk, d, int(causal),
                                         float(scale), DTYPE_CODES[dtype], b - a,
                                         _ptr(rb[a:b], _lp), _ptr(rr[a:b], _lp),
                                         _ptr(lse_sel[a:b]), _ptr(D_sel[a:b]))

    for rc in _threaded(rb.size, threads, stats):
        _check(rc, "fa_ref_bwd_rowstats_f64")
    lse_all[rb * Nq + rr] = lse_sel
    D_all[rb * Nq + rr] = D_sel
    dk, dv = np.empty((sel_bh.size, d)), np.empty((sel_bh.size, d))

    def keys(span):
        a, b = span
        if b <= a:
            return 0
        return L.fa_ref_bwd_dkv_keys_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                         dout.ctypes.data, B, H, Nq, Nk, d, int(causal),
                                         float(scale), DTYPE_CODES[dtype], _ptr(lse_all),
                                         _ptr(D_all), b - a, _ptr(sel_bh[a:b], _lp),
                                         _ptr(sel_key[a:b], _lp), _ptr(dk[a:b]), _ptr(dv[a:b]))

    for rc in _threaded(sel_bh.size, threads, keys):
        _check(rc, "fa_ref_bwd_dkv_keys_f64")
    return dk, dv


def bwd_ref(q, k, v, dout, causal: bool, scale: float, dtype: str, L=None):
    """Whole-tensor host backward: dq, dk, dv in the input dtype (RNE from fp64)."""
    L = L or lib()
    q, k, v, dout, B, H, Nq, Nk, d = _raw4(q, k, v, dout, dtype)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    _check(L.fa_bwd_ref(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                        dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, B, H, Nq, Nk, d,
                        int(causal), float(scale), DTYPE_CODES[dtype]), "fa_bwd_ref")
    return dq, dk, dv


# ---------------------------------------------------------------------------
# dropout (part 4): Philox4x32-10 and dropout on P
# ---------------------------------------------------------------------------

def philox4x32_10(ctr, key, L=None):
    """One Philox4x32-10 block: four 32-bit counter words, two key words -> four words."""
    L = L or lib()
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    out = (ctypes.c_uint32 * 4)()
    _check(L.fa_oracle_philox4x32_10(c, k, out), "fa_oracle_philox4x32_10")
    return [int(x) for x in out]


def dropout_keep(seed: int, t: int, bh: int, nq: int, nk: int, L=None) -> np.ndarray:
    """[nq, nk] uint8: 1 where element (q, k) of head bh is kept."""
    L = L or lib()
    keep = np.empty((nq, nk), dtype=np.uint8)
    _check(L.fa_oracle_dropout_keep(int(seed), int(t), int(bh), nq, nk, keep.ctypes.data),
           "fa_oracle_dropout_keep")
    return keep


def attention_dropout_f64(q, k, v, causal: bool, scale: float, t: int, seed: int, bh: int = 0,
                          rows=None, L=None):
    """Part 1 with dropout on P (one head of fp64 inputs); returns (o, lse)."""
    L = L or lib()
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, d = q.shape
    nk = k.shape[0]
    rows = np.arange(nq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    o = np.empty((rows.size, d))
    lse = np.empty(rows.size)
    _check(L.fa_oracle_attention_dropout_f64(_ptr(q), _ptr(k), _ptr(v), nq, nk, d, int(causal),
                                             float(scale), int(t), int(seed), int(bh), rows.size,
                                             _ptr(rows, _lp), _ptr(o), _ptr(lse)),
           "fa_oracle_attention_dropout_f64")
    return o, lse


def attention_bwd_dropout_f64(q, k, v, dout, causal: bool, scale: float, t: int, seed: int,
                              bh: int = 0, L=None):
    """Part 3 with dropout on P (one head of fp64 inputs); returns (dq, dk, dv)."""
    L = L or lib()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    nq, d = q.shape
    nk = k.shape[0]
    dq, dk, dv = np.empty((nq, d)), np.empty((nk, d)), np.empty((nk, d))
    _check(L.fa_oracle_attention_bwd_dropout_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), nq, nk,
                                                 d, int(causal), float(scale), int(t), int(seed),
                                                 int(bh), _ptr(dq), _ptr(dk), _ptr(dv)),
           "fa_oracle_attention_bwd_dropout_f64")
    return dq, dk, dv


def ref_rows_dropout_f64(q, k, v, causal: bool, scale: float, dtype: str, t: int, seed: int,
                         sel_bh, sel_row, threads: int | None = None, L=None):
    """Part 1 with dropout on selected rows of raw buffers (threaded); (o64, lse64)."""
    L = L or lib()
    q, k, v = _raw(q, dtype), _raw(k, dtype), _raw(v, dtype)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    sel_bh = np.ascontiguousarray(sel_bh, np.int64)
    sel_row = np.ascontiguousarray(sel_row, np.int64)
    o, lse = np.empty((sel_bh.size, d)), np.empty(sel_bh.size)

    def work(span):
        a, b = span
        if b <= a:
            return 0
        return L.fa_ref_rows_dropout_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Nq, Nk,
                                         d, int(causal), float(scale), DTYPE_CODES[dtype], int(t),
                                         int(seed), b - a, _ptr(sel_bh[a:b], _lp),
                                         _ptr(sel_row[a:b], _lp), _ptr(o[a:b]), _ptr(lse[a:b]))

    for rc in _threaded(sel_bh.size, threads, work):
        _check(rc, "fa_ref_rows_dropout_f64")
    return o, lse


def bwd_head_dropout_f64(q, k, v, dout, causal: bool, scale: float, dtype: str, t: int,
                         seed: int, bh: int, L=None):
    """Part 3 with dropout on head bh of raw buffers; returns fp64 (dq, dk, dv)."""
    L = L or lib()
    q, k, v, dout, B, H, Nq, Nk, d = _raw4(q, k, v, dout, dtype)
    dq, dk, dv = np.empty((Nq, d)), np.empty((Nk, d)), np.empty((Nk, d))
    _check(L.fa_ref_bwd_head_dropout_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                         dout.ctypes.data, B, H, Nq, Nk, d, int(causal),
                                         float(scale), DTYPE_CODES[dtype], int(t), int(seed),
                                         int(bh), _ptr(dq), _ptr(dk), _ptr(dv)),
           "fa_ref_bwd_head_dropout_f64")
    return dq, dk, dv


def fwd_ref(q, k, v, causal: bool, scale: float, dtype: str, L=None):
    """Whole-tensor host reference: o in the input dtype (RNE from fp64), lse fp32."""
    L = L or lib()
    q, k, v = _raw(q, dtype), _raw(k, dtype), _raw(v, dtype)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    o = np.empty((B, H, Nq, d), dtype=q.dtype)
    lse = np.empty((B, H, Nq), dtype=np.float32)
    _check(L.fa_fwd_ref(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                        lse.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), B, H, Nq, Nk, d,
                        int(causal), float(scale), DTYPE_CODES[dtype]), "fa_fwd_ref")
    return o, lse


def round_to(x, dtype: str, L=None) -> np.ndarray:
    """fp64 -> dtype storage with round-to-nearest-even (fa_fwd_ref's rounding)."""
    L = L or lib()
    x = _f64(x).ravel()
    out = np.empty(x.size, dtype={"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype])
    _check(L.fa_oracle_round(_ptr(x), x.size, DTYPE_CODES[dtype], out.ctypes.data),
           "fa_oracle_round")
    return out


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to fp64 (bf16 given as uint16 bit patterns)."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)
