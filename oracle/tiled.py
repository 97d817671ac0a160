"""The pages' tiled loop orders and a pure-Python naive row — TEST INFRASTRUCTURE.

These exist to show, by brute force on tiny inputs, that both published loop
orders reach the plain definition for EVERY way of cutting queries and keys into
contiguous blocks.  They are written from the algorithms' descriptions, in fp64
numpy, one head at a time:

* :func:`q_outer` — the order of the "05_flash_attention.py" course file's
  ``flash_attention_forward``: per query block an empty running state, which absorbs
  the key blocks left to right (skipping those wholly in the causal future) by the
  running-softmax recurrence — the new maximum, the old sums carried over by
  exp(old max - new max), the block's exponentials added — and finally O = o~ / d and
  L = m + log d.  The state is the blog page's (m, d, o~) triple, one row per query.
* :func:`kv_outer` — "Flash Attention" blog page, Algorithm 1: keys outside, queries
  inside; O, l, m live in "HBM" arrays and O is kept normalised after every step:
  m~ = rowmax S, P~ = exp(S - m~), l~ = rowsum P~, m_new = max(m, m~),
  l_new = e^{m - m_new} l + e^{m~ - m_new} l~,
  O <- diag(l_new)^-1 (diag(l) e^{m - m_new} O + e^{m~ - m_new} P~ V).
  Algorithm 1 omits tau and the mask; Algorithm 2 adds them (S = tau Q K^T, masked).
* :func:`naive_row_fsum` — the definition for one query row in pure Python with
  ``math.exp`` and correctly rounded sums (``math.fsum``).

Reading taken where the pages are silent: a row of a (query block, key block) pair
that is entirely masked contributes nothing; written as "skip the update for such
rows" so that (-inf) - (-inf) never occurs (the course file relies on key block 0
being visible to every query; Algorithm 1 with a mask needs the same guard).
"""
from __future__ import annotations

import functools
import math

import numpy as np


def _bounds(n: int, cuts) -> list[tuple[int, int]]:
    """Contiguous blocks of range(n) cut at the sorted interior positions ``cuts``."""
    edges = [0, *sorted(cuts), n]
    return [(edges[i], edges[i + 1]) for i in range(len(edges) - 1)]


def _mask(s: np.ndarray, qs: int, ks: int, causal: bool) -> np.ndarray:
    if not causal:
        return s
    qi = np.arange(qs, qs + s.shape[0])[:, None]
    kj = np.arange(ks, ks + s.shape[1])[None, :]
    return np.where(kj > qi, -np.inf, s)


def _absorb(state: np.ndarray, s: np.ndarray, v: np.ndarray) -> np.ndarray:
    """One step of the running-softmax recurrence for a block of query rows.

    state [rows, 2 + dim] holds (m, d, o~) per row: the largest score seen, the sum of
    exp(score - m) and the value rows weighted by the same exponentials.  s [rows, keys]
    are the block's scaled scores (-inf where masked), v [keys, dim] its value rows.
    The new largest score m' = max(m, max s); the old sums are carried over by the
    factor exp(m - m') and the block adds exp(s - m') and exp(s - m') v.  A row that
    sees no key of the block keeps its state (so (-inf) - (-inf) never occurs)."""
    m_old, d_old, o_old = state[:, 0], state[:, 1], state[:, 2:]
    seen = np.isfinite(s).any(axis=1)
    m_new = np.where(seen, np.maximum(m_old, s.max(axis=1)), m_old)
    carry = np.where(np.isfinite(m_old), np.exp(m_old - np.where(seen, m_new, 0.0)), 0.0)
    carry = np.where(seen, carry, 1.0)
    w = np.where(seen[:, None], np.exp(s - np.where(seen, m_new, 0.0)[:, None]), 0.0)
    out = np.empty_like(state)
    out[:, 0] = m_new
    out[:, 1] = carry * d_old + w.sum(axis=1)
    out[:, 2:] = carry[:, None] * o_old + w @ v
    return out


def q_outer(Q, K, V, causal: bool, scale: float, q_cuts=(), k_cuts=()):
    """Course-file order: query blocks outside, key blocks inside, state on chip.

    Each query block starts from the empty state (m = -inf, d = 0, o~ = 0) and absorbs
    the key blocks left to right (:func:`_absorb`); with the causal mask, key blocks
    that start after the block's last query hold no visible key and are not visited.
    At the end O = o~ / d and L = m + log d."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    n, dim = Q.shape
    key_blocks = _bounds(K.shape[0], k_cuts)
    out = np.empty((n, dim))
    lse = np.empty(n)
    for lo, hi in _bounds(n, q_cuts):
        state = np.zeros((hi - lo, 2 + dim))
        state[:, 0] = -np.inf
        todo = [(a, b) for a, b in key_blocks if not (causal and a >= hi)]
        state = functools.reduce(
            lambda st, kb: _absorb(st, _mask(Q[lo:hi] @ K[kb[0]:kb[1]].T * scale, lo, kb[0],
                                             causal), V[kb[0]:kb[1]]),
            todo, state)
        out[lo:hi] = state[:, 2:] / state[:, 1:2]
        lse[lo:hi] = state[:, 0] + np.log(state[:, 1])
    return out, lse


def kv_outer(Q, K, V, causal: bool, scale: float, q_cuts=(), k_cuts=()):
    """Blog Algorithm 1/2 order: key blocks outside, query blocks inside, state in 'HBM'."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    n, d = Q.shape
    m_total = K.shape[0]
    O = np.zeros((n, d))    # HBM
    ell = np.zeros(n)       # HBM
    m = np.full(n, -np.inf)  # HBM
    for ks, ke in _bounds(m_total, k_cuts):
        Kj, Vj = K[ks:ke], V[ks:ke]
        for qs, qe in _bounds(n, q_cuts):
            Oi, li, mi = O[qs:qe].copy(), ell[qs:qe].copy(), m[qs:qe].copy()
            S = _mask(Q[qs:qe] @ Kj.T * scale, qs, ks, causal)
            m_t = S.max(axis=1)
            live = np.isfinite(m_t)
            if not live.any():
                continue
            P_t = np.where(live[:, None], np.exp(S - np.where(live, m_t, 0.0)[:, None]), 0.0)
            l_t = P_t.sum(axis=1)
            m_new = np.where(live, np.maximum(mi, m_t), mi)
            a_old = np.where(np.isfinite(mi), np.exp(mi - m_new), 0.0)
            a_new = np.where(live, np.exp(m_t - m_new), 0.0)
            l_new = a_old * li + a_new * l_t
            upd = live
            Onew = ((li * a_old)[:, None] * Oi + a_new[:, None] * (P_t @ Vj)) / np.where(
                upd, l_new, 1.0)[:, None]
            O[qs:qe] = np.where(upd[:, None], Onew, Oi)
            ell[qs:qe] = np.where(upd, l_new, li)
            m[qs:qe] = m_new
    return O, m + np.log(ell)


def naive_row_fsum(q_row, K, V, r: int, causal: bool, scale: float):
    """One query row of the definition in pure Python; returns (o list, lse)."""
    q_row = [float(x) for x in q_row]
    s = []
    for kk in range(len(K)):
        if causal and kk > r:
            continue
        s.append((kk, scale * math.fsum(a * float(b) for a, b in zip(q_row, K[kk]))))
    m = max(x for _, x in s)
    e = [(kk, math.exp(x - m)) for kk, x in s]
    ell = math.fsum(w for _, w in e)
    d = len(q_row)
    o = [math.fsum(w * float(V[kk][t]) for kk, w in e) / ell for t in range(d)]
    return o, m + math.log(ell)
