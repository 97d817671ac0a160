"""Per-element error bounds of the GPU gradients, built from the ingredients.

The pages state no tolerance for the backward pass; this one follows from the GPU
path's arithmetic.  The gradients are sums of products whose factors are rounded to
the input dtype (unit roundoff u = 2^-8 for bf16, 2^-11 for fp16) before the MFMAs:
P (for dV) and dS = P o (dP - D) (for dQ and dK), with D taken from the stored,
rounded O; the fp32 accumulation and the exp2 of the scores add far less.  So every
element of a gradient G = sum_n a_n b_n can be off by about u times sum_n |a_n b_n|
besides the rounding of G itself:

    |G_gpu - G_ref| <= c u (|G_ref| + A),

with A the sum of the magnitudes of the products that make up that element:

    dV[j, t]:  A = sum_i P[i, j] Z[i, j] |dO[i, t]|
    dQ[i, t]:  A = scale sum_j |dS|[i, j] |K[j, t]|
    dK[j, t]:  A = scale sum_i |dS|[i, j] |Q[i, t]|
    |dS|[i, j] = P[i, j] (|dP[i, j]| Z[i, j] + sum_t |dO[i, t] O[i, t]|),  dP = dO V^T,
    O = (P o Z) V

(Z is the dropout factor, 1 without dropout; the last sum bounds D_i = dO_i . O_i and
the error of D from the rounded O).  fp16 adds an absolute floor: a factor smaller
than 2^-14 is rounded to a subnormal, off by up to eta = 2^-25 whatever its size, and
so is a small output; so the bound is

    |G_gpu - G_ref| <= c (u (|G_ref| + A) + eta (1 + F)),

F the sum of the magnitudes of the other factors of the element's products
(dV: sum_i Z[i, j] |dO[i, t]| over the rows that see key j; dQ: scale sum_j |K[j, t]|
over the keys row i sees; dK: scale sum_i |Q[i, t]| over the rows that see key j);
eta = 2^-134 for bf16 makes it vanish there.  The factors are computed here in fp64
from the same inputs, only to size the bound; the expected values come from the
oracle.  The tests print the largest |G_gpu - G_ref| / (u (|G_ref| + A)) they meet and
assert it stays below C (a few times the measured values).
"""
import numpy as np

import oracle

U = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
ETA = {"bf16": 2.0 ** -134, "f16": 2.0 ** -25}
C = 3.0


def _probs(qh, kh, causal, scale, vis=None, q_rows=None):
    """Softmax rows P[rows, :] of one head (fp64; rows with no visible key are 0) and the
    visibility of each (row, key)."""
    rows = np.arange(qh.shape[0]) if q_rows is None else np.asarray(q_rows)
    s = scale * (qh[rows] @ kh.T)
    hid = np.zeros(s.shape, bool)
    if causal:
        hid |= np.arange(kh.shape[0])[None, :] > rows[:, None]
    if vis is not None:
        hid |= ~vis[rows]
    s = np.where(hid, -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    live = np.isfinite(m[:, 0])
    e = np.exp(s - np.where(np.isfinite(m), m, 0.0))
    e[~live] = 0.0
    den = e.sum(axis=1, keepdims=True)
    return np.divide(e, den, out=np.zeros_like(e), where=den > 0), ~hid


def scales(w, q, k, v, dout, bh, vis=None, z=None, q_rows=None, k_cols=None):
    """Ingredient magnitudes A of dQ (rows q_rows, default all), dK and dV (keys k_cols,
    default all) of head bh.  vis: boolean [Nq, Nk] caller mask of the head; z: dropout
    factors [Nq, Nk] of the head."""
    qh, kh, vh, doh = (oracle.widen(a, w.dtype).reshape(w.B * w.H, -1, w.d)[bh]
                       for a in (q, k, v, dout))
    out = []
    # dQ rows: their own P rows over every key
    rq = np.arange(w.Nq) if q_rows is None else np.asarray(q_rows)
    P, seen = _probs(qh, kh, w.causal, w.scale, vis, rq)
    Zq = 1.0 if z is None else z[rq]
    dP = doh[rq] @ vh.T
    Dabs = (np.abs(doh[rq]) * np.abs((P * Zq) @ vh)).sum(axis=1, keepdims=True)
    aS = P * (np.abs(dP) * Zq + Dabs)
    out.append((w.scale * aS @ np.abs(kh), w.scale * seen @ np.abs(kh)))
    # dK, dV keys: every row's P in their columns
    kc = np.arange(w.Nk) if k_cols is None else np.asarray(k_cols)
    Pa, seen_a = _probs(qh, kh, w.causal, w.scale, vis)
    Za = 1.0 if z is None else z
    dPa = doh @ vh.T
    Dabs_a = (np.abs(doh) * np.abs((Pa * Za) @ vh)).sum(axis=1, keepdims=True)
    aSa = (Pa * (np.abs(dPa) * Za + Dabs_a))[:, kc]
    sk = seen_a[:, kc].astype(np.float64)
    out.append((w.scale * aSa.T @ np.abs(qh), w.scale * sk.T @ np.abs(qh)))
    out.append((((Pa * Za)[:, kc]).T @ np.abs(doh), ((seen_a * Za)[:, kc]).T @ np.abs(doh)))
    return out


def check(name, got64, ref64, af, dtype, say=print, c=C):
    """|got - ref| <= c (u (|ref| + A) + eta (1 + F)) element by element, af = (A, F) as
    scales() returns them; returns the largest ratio."""
    u = U[dtype]
    a, f = af
    assert np.isfinite(got64).all(), f"{name}: non-finite gradient"
    err = np.abs(got64 - ref64)
    lim = u * (np.abs(ref64) + a) + ETA[dtype] * (1.0 + f)
    ratio = np.divide(err, lim, out=np.where(err > 0, np.inf, 0.0), where=lim > 0)
    worst = float(ratio.max()) if ratio.size else 0.0
    say(f"    {name}: max |d| / bound = {worst:.3f}  max|d|={err.max() if err.size else 0:.3e}")
    assert worst <= c, f"{name}: element error {worst:.3f} x (u (|ref| + A) + eta (1 + F)) > {c}"
    return worst
