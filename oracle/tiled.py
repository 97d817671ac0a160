"""The pages' tiled loop orders and a pure-Python naive row — TEST INFRASTRUCTURE.

These exist to show, by brute force on tiny inputs, that both published loop
orders reach the plain definition for EVERY way of cutting queries and keys into
contiguous blocks.  They are written from the algorithms' descriptions, in fp64
numpy, one head at a time:

* :func:`q_outer` — "05_flash_attention.py" course file, ``flash_attention_forward``:
  per query block, state O~ = 0, m = -inf, l = 0; per key block (left to right,
  skipping blocks wholly in the causal future), S = Q_i K_j^T * scale, mask,
  m_new = max(m, rowmax S), P = exp(S - m_new), c = exp(m - m_new),
  l = c l + rowsum P, O~ = c O~ + P V_j, m = m_new; finally O = O~ / l and
  L = m + log l.
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


def q_outer(Q, K, V, causal: bool, scale: float, q_cuts=(), k_cuts=()):
    """Course-file order: query blocks outside, key blocks inside, state on chip."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    n, d = Q.shape
    m_total = K.shape[0]
    O = np.zeros((n, d))
    L = np.zeros(n)
    for qs, qe in _bounds(n, q_cuts):
        Oi = np.zeros((qe - qs, d))
        mi = np.full(qe - qs, -np.inf)
        li = np.zeros(qe - qs)
        for ks, ke in _bounds(m_total, k_cuts):
            if causal and ks > qe - 1:
                break  # the whole key block lies in the future of every query here
            S = _mask(Q[qs:qe] @ K[ks:ke].T * scale, qs, ks, causal)
            live = np.isfinite(S.max(axis=1))  # rows with at least one visible key
            m_new = np.where(live, np.maximum(mi, S.max(axis=1)), mi)
            P = np.where(live[:, None], np.exp(S - m_new[:, None]), 0.0)
            c = np.where(live & np.isfinite(mi), np.exp(mi - m_new), np.where(live, 0.0, 1.0))
            li = c * li + P.sum(axis=1)
            Oi = c[:, None] * Oi + P @ V[ks:ke]
            mi = m_new
        O[qs:qe] = Oi / li[:, None]
        L[qs:qe] = mi + np.log(li)
    return O, L


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
