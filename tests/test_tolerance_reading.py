"""The reading of the bf16 max bound, checked on the CPU by emulating the arithmetic.

The stated bound for bf16 outputs is max |dO| <= 1e-2.  Where |O_ref| >= 4 one bf16
step is 2^-5, so correct rounding of the output alone can miss O_ref by up to 2^-6 >
1e-2; there an element passes if it is one of the two bf16 neighbours of O_ref.  Below
4 the literal bound is applied.  This file shows, with fp32 emulations of the
arithmetic in numpy (no GPU), that the literal bound below 4 is reachable by the
method the pages describe and by the rule the kernels use:

* the pages' recurrence (course page "05_flash_attention.py", flash_attention_forward:
  running max per key tile, P = exp(S - m_new), l = c l + rowsum P, O~ = c O~ + P V,
  O = O~ / l), with P rounded to bf16 for the P.V product as the article on hncyxsy.com
  casts it (section 5.4) and everything else in fp32;
* the kernels' rule: exp2 with the scale folded in, a reference max that moves to the
  rows' maxima when a key would weigh more than 1/5 of its row (tested per wave of 32
  rows and per half-row of keys, the threshold refreshed every second tile), and O
  divided by the sum of the rounded P that entered the P.V product;
* the former kernel rule (reference moved only 2^8 above the row max) as the contrast:
  it leaves a row's dominant weight rounded, and on these seeds it exceeds 1e-2 on
  elements with 2 <= |O_ref| < 4.

The pages' recurrence divides by the sum of the fp32 P while the rounded P multiplies V;
on one of the seeds that alone misses 1e-2 on a few elements of the band, which is why
the kernels divide by the sum of the rounded P (the weights that multiply V then sum
to one).

The inputs are three shapes of the GPU sweep with logits of standard deviation 9 (Q and
K drawn with sigma 3), the regime where rows are peaked and |O| reaches 2-4.
"""
import numpy as np
import pytest

import oracle
from flashattention_tiling_online_amd import inputs
from sweep_specs import FWD, workload

SPECS = {s[0]: s for s in FWD}
CASES = ["s7_11", "s7_20", "s7_45"]
LOG2E = 1.4426950408889634


def bf16(x):
    """fp32 -> bf16 (nearest-even) -> fp32 values."""
    bits = inputs.round_fp32(np.ascontiguousarray(x, dtype=np.float32), "bf16")
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _half_of_key(nk):
    """Half (0 or 1) of a 64-key tile that owns each key in the kernels' layout: key
    offsets 8 g + 4 h + 0..3 of every 8-key group belong to half h."""
    return (np.arange(nk) % 8) // 4


def emulate(q, k, v, causal, scale, rule):
    """One head in fp32, keys in tiles of 64.  rule: 'pages', 'kernel' or 'lazy8'."""
    nq, nk = q.shape[0], k.shape[0]
    s_raw = (q.astype(np.float64) @ k.astype(np.float64).T).astype(np.float32)
    if causal:
        s_raw = np.where(np.arange(nk)[None, :] > np.arange(nq)[:, None], -np.inf, s_raw)
    o = np.zeros((nq, q.shape[1]), np.float32)
    l = np.zeros(nq, np.float32)       # sum of the fp32 P
    lr = np.zeros(nq, np.float32)      # sum of the rounded P
    if rule == "pages":
        m = np.full(nq, -np.inf, np.float32)
        for t0 in range(0, nk, 64):
            st = (s_raw[:, t0:t0 + 64] * np.float32(scale)).astype(np.float32)
            m_new = np.maximum(m, st.max(axis=1))
            live = np.isfinite(m_new)
            c = np.where(np.isfinite(m), np.exp(m - np.where(live, m_new, 0)), 0).astype(np.float32)
            p = np.where(np.isfinite(st), np.exp(st - np.where(live, m_new, 0)[:, None]), 0)
            p = p.astype(np.float32)
            l = (c * l + p.sum(axis=1, dtype=np.float32)).astype(np.float32)
            o = (c[:, None] * o + (bf16(p).astype(np.float64) @ v[t0:t0 + 64]).astype(np.float32))
            o = o.astype(np.float32)
            m = np.where(live, m_new, m).astype(np.float32)
        return bf16(o / l[:, None]).astype(np.float64)
    # base-2 forms: s c2 - m2 in one rounding (a fused multiply-add), P = 2^(...)
    c2 = np.float32(np.float32(scale) * np.float32(LOG2E))
    m2 = np.full(nq, -np.inf, np.float32)
    thr = np.full((nq, 2), -np.inf, np.float32)   # per row and half, in log2 units
    half = _half_of_key(min(nk, 64))
    lh = np.zeros((nq, 2), np.float32)           # the halves' fp32 sums
    for j, t0 in enumerate(range(0, nk, 64)):
        st = s_raw[:, t0:t0 + 64]
        hm = np.stack([(st[:, half[:st.shape[1]] == h].max(axis=1, initial=-np.inf)
                        * np.float64(c2)).astype(np.float32) for h in (0, 1)], axis=1)
        trig = (hm > thr).any(axis=1)
        move = np.zeros(nq, bool)
        for w0 in range(0, nq, 32):                 # the decision is per wave of 32 rows
            move[w0:w0 + 32] = trig[w0:w0 + 32].any()
        m_new = np.where(move, np.maximum(m2, hm.max(axis=1)), m2).astype(np.float32)
        alpha = np.where(move & np.isfinite(m2), np.exp2(m2 - np.where(np.isfinite(m_new), m_new, 0)),
                         np.where(move, 0, 1)).astype(np.float32)
        alpha = np.where(np.isfinite(m_new) | ~move, alpha, 1).astype(np.float32)
        o, l, lr = o * alpha[:, None], l * alpha, lr * alpha
        lh = lh * alpha[:, None]
        m2 = m_new
        mm = np.where(np.isfinite(m2), m2, 0).astype(np.float64)
        arg = (st.astype(np.float64) * np.float64(c2) - mm[:, None]).astype(np.float32)
        p = np.where(np.isfinite(st), np.exp2(arg), 0).astype(np.float32)
        pr = bf16(p)
        l = (l + p.sum(axis=1, dtype=np.float32)).astype(np.float32)
        lr = (lr + pr.sum(axis=1, dtype=np.float32)).astype(np.float32)
        for h in (0, 1):
            lh[:, h] += p[:, half[:st.shape[1]] == h].sum(axis=1, dtype=np.float32)
        o = (o + (pr.astype(np.float64) @ v[t0:t0 + 64]).astype(np.float32)).astype(np.float32)
        if rule == "lazy8":
            thr = np.repeat((m2 + 8)[:, None], 2, axis=1).astype(np.float32)
        else:
            thr = np.where(move[:, None], m2[:, None], thr)
            if j % 2 == 1:
                e = np.frexp(lh)[1]
                thr = (m2[:, None] + np.clip(e - 3, 0, 8)).astype(np.float32)
        thr = np.where(np.isfinite(m2)[:, None], thr, -np.inf).astype(np.float32)
    return bf16(o / lr[:, None]).astype(np.float64)


def _case(name):
    w = workload(SPECS[name])
    q, k, v = inputs.make_qkv(w)
    bh = np.repeat(np.arange(w.B * w.H), w.Nq)
    rows = np.tile(np.arange(w.Nq), w.B * w.H)
    o64, _ = oracle.ref_rows_f64(q, k, v, w.causal, w.scale, w.dtype, bh, rows)
    heads = [tuple(oracle.widen(a, "bf16").reshape(w.B * w.H, -1, w.d)[i].astype(np.float32)
                   for a in (q, k, v)) for i in range(w.B * w.H)]
    return w, heads, o64.reshape(w.B * w.H, w.Nq, w.d)


@pytest.fixture(scope="module")
def cases():
    return {n: _case(n) for n in CASES}


def _errors(w, heads, o64, rule):
    out = np.stack([emulate(qh, kh, vh, w.causal, w.scale, rule) for qh, kh, vh in heads])
    return np.abs(out - o64), np.abs(o64)


def test_cases_are_peaked(cases):
    for name, (w, _, o64) in cases.items():
        assert w.dtype == "bf16" and w.sigma_q == 3.0
        assert np.abs(o64).max() >= 2.0, name   # the band 2 <= |O| < 4 is reached


@pytest.mark.parametrize("name", CASES)
def test_kernel_rule_meets_literal_bound_below_4(cases, name):
    w, heads, o64 = cases[name]
    err, mag = _errors(w, heads, o64, "kernel")
    assert err[mag < 4].max() <= 1e-2, err[mag < 4].max()
    assert err.mean() <= 1e-3


@pytest.mark.parametrize("name", ["s7_20", "s7_45"])
def test_pages_recurrence_meets_literal_bound_below_4(cases, name):
    w, heads, o64 = cases[name]
    err, mag = _errors(w, heads, o64, "pages")
    assert err[mag < 4].max() <= 1e-2, err[mag < 4].max()


def test_lazy_reference_exceeds_literal_bound(cases):
    """The former rule leaves the dominant weight rounded: over these seeds some element
    with 2 <= |O_ref| < 4 misses by more than 1e-2, which the rules above avoid."""
    over = 0
    for name, (w, heads, o64) in cases.items():
        err, mag = _errors(w, heads, o64, "lazy8")
        over += int(((err > 1e-2) & (mag >= 2) & (mag < 4)).sum())
    assert over >= 1


def test_pages_recurrence_with_fp32_sum_can_exceed(cases):
    """Dividing by the fp32 sum while V is weighted by the rounded P leaves the weights
    summing to 1 + O(2^-9): on s7_11 that misses 1e-2 on elements of the band."""
    w, heads, o64 = cases["s7_11"]
    err, mag = _errors(w, heads, o64, "pages")
    assert int(((err > 1e-2) & (mag >= 2) & (mag < 4)).sum()) >= 1
