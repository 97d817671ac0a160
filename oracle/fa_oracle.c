/*
 * fa_oracle.c — fp64 CPU oracle for the fused attention forward pass and its gradients.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this code.  The GPU library shares nothing with it.
 *
 * It is deliberately plain: loops in the order the definitions are written, fp64,
 * left-to-right sums, no blocking, no fusion, no reordering.  Build flags keep
 * IEEE semantics (no fast-math, no FMA contraction).
 *
 * What it follows (the pages are named by their titles / addresses):
 *   [A] "05_flash_attention.py" (CS336 lecture-5 course file, semidirectx.com):
 *       standard_attention (scale, causal triu mask, softmax, @V),
 *       flash_attention_forward (returned L = m + log l), online_softmax_stats,
 *       flash_attention_backward (the gradient formulas of part 3).
 *   [B] "Flash Attention" (blog.cyberangel.work): sections "Online Softmax"
 *       (safe softmax, the online recurrence and its invariant), the parallelisation
 *       section (the (+) operator on (m, d) and on (m, d, o~)), Algorithm 2 (tau, mask),
 *       Algorithm 4 (backward pass) and the softmax-Jacobian derivation after it.
 *   [C] "手写 Flash Attention：从算法原理到高性能实现" (bjdmk.com.cn), section 2.2:
 *       the worked two-block example that the tests pin.
 *   [D] Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 *       easy as 1, 2, 3", SC'11): the random numbers of dropout, which [B] leaves
 *       unspecified.
 * Parts: 1 three-step attention, 2 the online accumulator and (+), 3 gradients,
 * 4 dropout, 5 caller masks (threaded through parts 1-3 as an optional mask row).
 *
 * Readings where the pages are silent are listed beside the code that takes them.
 */
#include "../include/fa_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* exact widening of the stored element types to fp64                        */
/* ------------------------------------------------------------------------- */

static double widen_bf16(uint16_t bits)
{
    /* bf16 is the upper half of an IEEE binary32 */
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double widen_f16(uint16_t bits)
{
    /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits */
    int sign = bits >> 15;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(frac | 0x400), expo - 25);
    return sign ? -mag : mag;
}

static double widen_one(const void* base, int64_t idx, int dtype)
{
    if (dtype == FA_ORACLE_F32) {
        float f;
        memcpy(&f, (const char*)base + 4 * idx, 4);
        return (double)f;
    }
    uint16_t h;
    memcpy(&h, (const char*)base + 2 * idx, 2);
    return dtype == FA_ORACLE_BF16 ? widen_bf16(h) : widen_f16(h);
}

static void widen_span(const void* base, int64_t first, int64_t count, int dtype, double* out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = widen_one(base, first + i, dtype);
}

/* ------------------------------------------------------------------------- */
/* one-dimensional online softmax with per-block trace  [B] "Online Softmax",  */
/* [A] online_softmax_stats                                                  */
/* ------------------------------------------------------------------------- */

int fa_oracle_softmax_online(const double* x, int64_t n, int64_t block, double* y,
                             double* run_m, double* run_l, double* carried, double* fresh)
{
    if (!x || n < 1 || block < 1)
        return FA_ORACLE_EINVAL;

    double m = -INFINITY; /* running maximum, starts at -inf */
    double l = 0.0;       /* running sum relative to m, starts at 0 */
    int64_t b = 0;
    for (int64_t start = 0; start < n; start += block, ++b) {
        int64_t end = start + block < n ? start + block : n;

        /* new maximum over the old one and the block */
        double m_new = m;
        for (int64_t i = start; i < end; ++i)
            if (x[i] > m_new)
                m_new = x[i];

        /* rebase the old sum to the new maximum; while nothing finite has been
         * read yet (m = m_new = -inf) there is nothing to carry */
        double carry = (l == 0.0) ? 0.0 : l * exp(m - m_new);

        /* the block's own contribution relative to the new maximum */
        double add = 0.0;
        if (m_new != -INFINITY)
            for (int64_t i = start; i < end; ++i)
                add += exp(x[i] - m_new);

        l = carry + add;
        m = m_new;
        if (run_m) run_m[b] = m;
        if (run_l) run_l[b] = l;
        if (carried) carried[b] = carry;
        if (fresh) fresh[b] = add;
    }
    if (m == -INFINITY)
        return FA_ORACLE_EINVAL; /* no finite value: softmax undefined */

    /* second pass: normalise with the final statistics */
    if (y)
        for (int64_t i = 0; i < n; ++i)
            y[i] = exp(x[i] - m) / l;
    return FA_ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* the (+) merge on (m, d, o~)  [B] parallelisation section                  */
/* ------------------------------------------------------------------------- */

int fa_oracle_merge(int64_t dim, const double* a, const double* b, double* out)
{
    if (!a || !b || !out || dim < 0)
        return FA_ORACLE_EINVAL;
    double ma = a[0], mb = b[0];
    /* The empty state (-inf, 0, 0) is the identity.  The pages leave
     * (-inf) - (-inf) undefined; returning the other operand is the reading that
     * makes the -inf initial state degenerate to plain softmax, as [A] and [C] say. */
    if (ma == -INFINITY || mb == -INFINITY) {
        const double* keep = (ma == -INFINITY) ? b : a;
        if (keep != out)
            memmove(out, keep, (size_t)(dim + 2) * sizeof(double));
        return FA_ORACLE_OK;
    }
    double m = ma > mb ? ma : mb;
    double ca = exp(ma - m);
    double cb = exp(mb - m);
    double d = a[1] * ca + b[1] * cb;
    for (int64_t t = 0; t < dim; ++t)
        out[2 + t] = a[2 + t] * ca + b[2 + t] * cb;
    out[0] = m;
    out[1] = d;
    return FA_ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Dropout on P and its random numbers                                        */
/*   [B] Algorithm 2 (P_dropped = dropout(P, p), O = P_dropped V; the forward  */
/*   returns the RNG state R) and Algorithm 4 (Z regenerated from R,          */
/*   P_dropped = P o Z, dP = dP_dropped o Z).  The pages name no generator;   */
/*   the reading taken here: Philox4x32-10, the counter-based generator of    */
/*   Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1,   */
/*   2, 3" (SC'11), with key = (seed low 32 bits, seed high 32 bits) and       */
/*   counter = (k / 4, q / 4, bh, 0) for element (bh, q, k); its 16 output     */
/*   bytes (word w, byte b = bits 8b..8b+7, index 4w + b) cover the 4x4 block  */
/*   of queries 4(q/4).. and keys 4(k/4)..: element (q, k) takes byte          */
/*   4 (q % 4) + k % 4.  The element is dropped iff that byte is below the     */
/*   threshold t (0 <= t < 256, the drop probability is t / 256) and kept      */
/*   values are scaled by 256 / (256 - t), so that E[Z] = 1.                   */
/* ------------------------------------------------------------------------- */

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

int fa_oracle_philox4x32_10(const uint32_t* ctr_in, const uint32_t* key_in, uint32_t* out)
{
    if (!ctr_in || !key_in || !out)
        return FA_ORACLE_EINVAL;
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { /* bump the key between rounds */
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        const uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
        const uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c[0] = n0;
        c[1] = n1;
        c[2] = n2;
        c[3] = n3;
    }
    for (int i = 0; i < 4; ++i)
        out[i] = c[i];
    return FA_ORACLE_OK;
}

typedef struct {
    uint64_t seed;
    int t;             /* drop iff byte < t */
    double keep_scale; /* 256 / (256 - t) */
    int64_t bh;
} Drop;

/* Z[q, k] of head dr->bh: 0 (dropped) or keep_scale; 1 without dropout (dr NULL) */
static double drop_factor(const Drop* dr, int64_t q, int64_t k)
{
    if (!dr)
        return 1.0;
    const uint32_t ctr[4] = {(uint32_t)(k >> 2), (uint32_t)(q >> 2), (uint32_t)dr->bh, 0u};
    const uint32_t key[2] = {(uint32_t)dr->seed, (uint32_t)(dr->seed >> 32)};
    uint32_t w[4];
    fa_oracle_philox4x32_10(ctr, key, w);
    const int idx = (int)(4 * (q & 3) + (k & 3));
    const uint32_t byte = (w[idx >> 2] >> (8 * (idx & 3))) & 0xFFu;
    return (int)byte < dr->t ? 0.0 : dr->keep_scale;
}

static int make_drop(Drop* dr, int t, uint64_t seed, int64_t bh)
{
    if (t < 0 || t > 255)
        return FA_ORACLE_EINVAL;
    dr->seed = seed;
    dr->t = t;
    dr->keep_scale = 256.0 / (256.0 - (double)t);
    dr->bh = bh;
    return FA_ORACLE_OK;
}

int fa_oracle_dropout_keep(uint64_t seed, int t, int64_t bh, int64_t nq, int64_t nk,
                           uint8_t* keep)
{
    Drop dr;
    if (!keep || nq < 0 || nk < 0 || bh < 0 || make_drop(&dr, t, seed, bh))
        return FA_ORACLE_EINVAL;
    for (int64_t q = 0; q < nq; ++q)
        for (int64_t k = 0; k < nk; ++k)
            keep[q * nk + k] = drop_factor(&dr, q, k) != 0.0;
    return FA_ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Part 1: standard three-step attention, one row  [A] standard_attention     */
/* ------------------------------------------------------------------------- */

/* ------------------------------------------------------------------------- */
/* Caller masks  [B] Algorithm 2 (S_masked = mask(S), P = softmax(S_masked)) and  */
/*   Algorithm 4 (the backward recomputes P from mask(S)).  Reading: mask(S)   */
/*   sets S[q, k] to -inf where the caller's boolean mask is false, as the     */
/*   course page's masked_fill does for its causal mask; the mask of one query */
/*   row is bit-packed, key k in bit k % 32 of 32-bit word k / 32 (bit set =   */
/*   visible).  A row with no visible key has no softmax: the reading taken is */
/*   O = 0 and L = -inf (the identity of the (+) merge), P = 0 in the backward.*/
/* ------------------------------------------------------------------------- */

/* is key kk visible in the caller's mask row mrow (NULL: no caller mask)? */
static int mask_visible(const uint32_t* mrow, int64_t kk)
{
    return !mrow || ((mrow[kk / 32] >> (kk % 32)) & 1u);
}

/* score of query row r against key kk: scale * sum_t q[t] k[t], or -inf if masked
 * (causal rule, then the caller's mask row mrow when given) */
static double score(const double* q_row, const double* k_row, int64_t d, double scale,
                    int causal, int64_t r, int64_t kk, const uint32_t* mrow)
{
    if (causal && kk > r)
        return -INFINITY;
    if (!mask_visible(mrow, kk))
        return -INFINITY;
    double dot = 0.0;
    for (int64_t t = 0; t < d; ++t)
        dot += q_row[t] * k_row[t];
    return scale * dot;
}

/* s is caller scratch of nk doubles */
static void three_step_row(const double* q_row, const double* k, const double* v, int64_t nk,
                           int64_t d, int causal, double scale, int64_t r, double* s,
                           double* o_row, double* lse, const Drop* dr, const uint32_t* mrow)
{
    /* step 1: materialise the score row S[r, :] */
    for (int64_t kk = 0; kk < nk; ++kk)
        s[kk] = score(q_row, k + kk * d, d, scale, causal, r, kk, mrow);

    /* step 2: safe softmax — maximum, shifted exponentials, sum, normalise */
    double m = -INFINITY;
    for (int64_t kk = 0; kk < nk; ++kk)
        if (s[kk] > m)
            m = s[kk];
    if (m == -INFINITY) { /* no visible key (caller mask): O = 0, L = -inf */
        for (int64_t t = 0; t < d; ++t)
            o_row[t] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int64_t kk = 0; kk < nk; ++kk) {
        s[kk] = exp(s[kk] - m); /* masked keys: exp(-inf) = 0 */
        l += s[kk];
    }
    for (int64_t kk = 0; kk < nk; ++kk)
        s[kk] = s[kk] / l; /* P[r, :] */

    /* step 3: O[r, :] = P_dropped[r, :] V, P_dropped = P o Z (Z = 1 without dropout) */
    for (int64_t t = 0; t < d; ++t)
        o_row[t] = 0.0;
    for (int64_t kk = 0; kk < nk; ++kk) {
        const double pk = s[kk] * drop_factor(dr, r, kk);
        for (int64_t t = 0; t < d; ++t)
            o_row[t] += pk * v[kk * d + t];
    }

    /* logsumexp of the scaled, masked scores */
    *lse = m + log(l);
}

int fa_oracle_attention_f64(const double* q, const double* k, const double* v,
                            int64_t nq, int64_t nk, int64_t d, int causal, double scale,
                            int64_t n_rows, const int64_t* rows, double* o, double* lse)
{
    if (!q || !k || !v || !o || !lse || nq < 1 || nk < 1 || d < 1 || n_rows < 0 ||
        (n_rows > 0 && !rows))
        return FA_ORACLE_EINVAL;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= nq)
            return FA_ORACLE_EINVAL;
    double* s = (double*)malloc((size_t)nk * sizeof(double));
    if (!s)
        return FA_ORACLE_ENOMEM;
    for (int64_t i = 0; i < n_rows; ++i)
        three_step_row(q + rows[i] * d, k, v, nk, d, causal, scale, rows[i], s, o + i * d,
                       lse + i, NULL, NULL);
    free(s);
    return FA_ORACLE_OK;
}

int fa_oracle_attention_dropout_f64(const double* q, const double* k, const double* v,
                                    int64_t nq, int64_t nk, int64_t d, int causal, double scale,
                                    int t, uint64_t seed, int64_t bh, int64_t n_rows,
                                    const int64_t* rows, double* o, double* lse)
{
    Drop dr;
    if (!q || !k || !v || !o || !lse || nq < 1 || nk < 1 || d < 1 || n_rows < 0 ||
        (n_rows > 0 && !rows) || bh < 0 || make_drop(&dr, t, seed, bh))
        return FA_ORACLE_EINVAL;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= nq)
            return FA_ORACLE_EINVAL;
    double* s = (double*)malloc((size_t)nk * sizeof(double));
    if (!s)
        return FA_ORACLE_ENOMEM;
    for (int64_t i = 0; i < n_rows; ++i)
        three_step_row(q + rows[i] * d, k, v, nk, d, causal, scale, rows[i], s, o + i * d,
                       lse + i, &dr, NULL);
    free(s);
    return FA_ORACLE_OK;
}

int fa_oracle_attention_masked_f64(const double* q, const double* k, const double* v,
                                   const uint32_t* mask_rows, int64_t nq, int64_t nk, int64_t d,
                                   int causal, double scale, int64_t n_rows, const int64_t* rows,
                                   double* o, double* lse)
{
    if (!q || !k || !v || !mask_rows || !o || !lse || nq < 1 || nk < 1 || d < 1 || n_rows < 0 ||
        (n_rows > 0 && !rows))
        return FA_ORACLE_EINVAL;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= nq)
            return FA_ORACLE_EINVAL;
    double* s = (double*)malloc((size_t)nk * sizeof(double));
    if (!s)
        return FA_ORACLE_ENOMEM;
    const int64_t W = (nk + 31) / 32;
    for (int64_t i = 0; i < n_rows; ++i)
        three_step_row(q + rows[i] * d, k, v, nk, d, causal, scale, rows[i], s, o + i * d,
                       lse + i, NULL, mask_rows + rows[i] * W);
    free(s);
    return FA_ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Part 2: scalar online (m, d, o~) accumulator  [B] "Online Softmax" and the  */
/* o~ extension; [A] flash_attention_forward for the returned L               */
/* ------------------------------------------------------------------------- */

/* State layout [m, d, o~_0..o~_{dim-1}], as for fa_oracle_merge. */

/* fold one visible key with score x and value row vrow into the state */
static void online_step(double* st, int64_t dim, double x, const double* vrow, int64_t* raised,
                        int first)
{
    double m_old = st[0];
    double m_new = x > m_old ? x : m_old;
    if (!first && m_new > m_old && raised)
        ++*raised;
    double c = first ? 0.0 : exp(m_old - m_new); /* rescale factor of the old state */
    double e = exp(x - m_new);                     /* weight of the new key */
    st[1] = st[1] * c + e;
    for (int64_t t = 0; t < dim; ++t)
        st[2 + t] = st[2 + t] * c + e * vrow[t];
    st[0] = m_new;
}

static void online_row(const double* q_row, const double* k, const double* v, int64_t nk,
                       int64_t d, int causal, double scale, int64_t r, int64_t key_block,
                       double* run, double* blk, double* o_row, double* lse, int64_t* raised,
                       const uint32_t* mrow)
{
    run[0] = -INFINITY;
    run[1] = 0.0;
    for (int64_t t = 0; t < d; ++t)
        run[2 + t] = 0.0;
    int64_t nraised = 0;
    int seen = 0; /* has the running state absorbed a visible key yet? */

    if (key_block <= 0) {
        for (int64_t kk = 0; kk < nk; ++kk) {
            double x = score(q_row, k + kk * d, d, scale, causal, r, kk, mrow);
            if (x == -INFINITY)
                continue; /* masked key: skipped */
            online_step(run, d, x, v + kk * d, &nraised, !seen);
            seen = 1;
        }
    } else {
        for (int64_t k0 = 0; k0 < nk; k0 += key_block) {
            int64_t k1 = k0 + key_block < nk ? k0 + key_block : nk;
            /* reduce the block to its own state, starting from the empty state */
            blk[0] = -INFINITY;
            blk[1] = 0.0;
            for (int64_t t = 0; t < d; ++t)
                blk[2 + t] = 0.0;
            int blk_seen = 0;
            for (int64_t kk = k0; kk < k1; ++kk) {
                double x = score(q_row, k + kk * d, d, scale, causal, r, kk, mrow);
                if (x == -INFINITY)
                    continue;
                online_step(blk, d, x, v + kk * d, NULL, !blk_seen);
                blk_seen = 1;
            }
            if (!blk_seen)
                continue; /* a fully masked block contributes the identity */
            if (seen && blk[0] > run[0])
                ++nraised;
            fa_oracle_merge(d, run, blk, run);
            seen = 1;
        }
    }
    /* final normalisation and logsumexp; a row that absorbed no key keeps the empty
     * state, read as O = 0 and L = -inf */
    for (int64_t t = 0; t < d; ++t)
        o_row[t] = seen ? run[2 + t] / run[1] : 0.0;
    *lse = seen ? run[0] + log(run[1]) : -INFINITY;
    if (raised)
        *raised = nraised;
}

int fa_oracle_online_f64(const double* q, const double* k, const double* v,
                         int64_t nq, int64_t nk, int64_t d, int causal, double scale,
                         int64_t key_block, int64_t n_rows, const int64_t* rows,
                         double* o, double* lse, int64_t* max_raised)
{
    if (!q || !k || !v || !o || !lse || nq < 1 || nk < 1 || d < 1 || n_rows < 0 ||
        (n_rows > 0 && !rows))
        return FA_ORACLE_EINVAL;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= nq)
            return FA_ORACLE_EINVAL;
    double* run = (double*)malloc((size_t)(2 * (d + 2)) * sizeof(double));
    if (!run)
        return FA_ORACLE_ENOMEM;
    double* blk = run + (d + 2);
    for (int64_t i = 0; i < n_rows; ++i)
        online_row(q + rows[i] * d, k, v, nk, d, causal, scale, rows[i], key_block, run, blk,
                   o + i * d, lse + i, max_raised ? max_raised + i : NULL, NULL);
    free(run);
    return FA_ORACLE_OK;
}

int fa_oracle_online_masked_f64(const double* q, const double* k, const double* v,
                                const uint32_t* mask_rows, int64_t nq, int64_t nk, int64_t d,
                                int causal, double scale, int64_t key_block, int64_t n_rows,
                                const int64_t* rows, double* o, double* lse)
{
    if (!q || !k || !v || !mask_rows || !o || !lse || nq < 1 || nk < 1 || d < 1 || n_rows < 0 ||
        (n_rows > 0 && !rows))
        return FA_ORACLE_EINVAL;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= nq)
            return FA_ORACLE_EINVAL;
    double* run = (double*)malloc((size_t)(2 * (d + 2)) * sizeof(double));
    if (!run)
        return FA_ORACLE_ENOMEM;
    const int64_t W = (nk + 31) / 32;
    for (int64_t i = 0; i < n_rows; ++i)
        online_row(q + rows[i] * d, k, v, nk, d, causal, scale, rows[i], key_block, run,
                   run + (d + 2), o + i * d, lse + i, NULL, mask_rows + rows[i] * W);
    free(run);
    return FA_ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* raw-buffer entry points                                                   */
/* ------------------------------------------------------------------------- */

static int check_raw(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                     int64_t Nq, int64_t Nk, int64_t d, int dtype)
{
    if (!q || !k || !v)
        return FA_ORACLE_EINVAL;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1)
        return FA_ORACLE_EINVAL;
    if (dtype != FA_ORACLE_F32 && dtype != FA_ORACLE_F16 && dtype != FA_ORACLE_BF16)
        return FA_ORACLE_EINVAL;
    return FA_ORACLE_OK;
}

/* shared driver of fa_ref_rows_f64 / fa_ref_online_f64: widens K and V once per run
 * of equal sel_bh, widens each selected query row, then runs part 1 or part 2 on it */
/* the caller-mask row of query r of head bh in a [mask_b, mask_h, Nq, W] array, W =
 * ceil(Nk / 32) words, whose leading extents are 1 (shared) or B and H */
static const uint32_t* mask_row(const uint32_t* mask, int64_t mask_b, int64_t mask_h, int64_t H,
                                int64_t Nq, int64_t Nk, int64_t bh, int64_t r)
{
    if (!mask)
        return NULL;
    const int64_t W = (Nk + 31) / 32;
    const int64_t b = mask_b == 1 ? 0 : bh / H, h = mask_h == 1 ? 0 : bh % H;
    return mask + ((b * mask_h + h) * Nq + r) * W;
}

static int check_mask(const uint32_t* mask, int64_t mask_b, int64_t mask_h, int64_t B, int64_t H)
{
    if (!mask)
        return FA_ORACLE_OK;
    if ((mask_b != 1 && mask_b != B) || (mask_h != 1 && mask_h != H))
        return FA_ORACLE_EINVAL;
    return FA_ORACLE_OK;
}

static int ref_rows(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                    int64_t Nq, int64_t Nk, int64_t d, int causal, float scale, int dtype,
                    int64_t n_sel, const int64_t* sel_bh, const int64_t* sel_row,
                    int use_online, int64_t key_block, double* o64, double* lse64,
                    int64_t* max_raised, int drop_t, uint64_t seed, const uint32_t* mask,
                    int64_t mask_b, int64_t mask_h)
{
    int rc = check_raw(q, k, v, B, H, Nq, Nk, d, dtype);
    if (rc)
        return rc;
    if (check_mask(mask, mask_b, mask_h, B, H))
        return FA_ORACLE_EINVAL;
    Drop dr;
    if (drop_t >= 0 && make_drop(&dr, drop_t, seed, 0))
        return FA_ORACLE_EINVAL;
    if (n_sel < 0 || (n_sel > 0 && (!sel_bh || !sel_row || !o64 || !lse64)))
        return FA_ORACLE_EINVAL;
    for (int64_t i = 0; i < n_sel; ++i)
        if (sel_bh[i] < 0 || sel_bh[i] >= B * H || sel_row[i] < 0 || sel_row[i] >= Nq)
            return FA_ORACLE_EINVAL;

    double* kh = (double*)malloc((size_t)(Nk * d) * sizeof(double));
    double* vh = (double*)malloc((size_t)(Nk * d) * sizeof(double));
    double* qr = (double*)malloc((size_t)d * sizeof(double));
    double* s = (double*)malloc((size_t)Nk * sizeof(double));
    double* st = (double*)malloc((size_t)(2 * (d + 2)) * sizeof(double));
    if (!kh || !vh || !qr || !s || !st) {
        free(kh);
        free(vh);
        free(qr);
        free(s);
        free(st);
        return FA_ORACLE_ENOMEM;
    }
    const double sc = (double)scale; /* the fp32 argument, widened exactly */
    int64_t cur = -1;
    for (int64_t i = 0; i < n_sel; ++i) {
        int64_t bh = sel_bh[i], r = sel_row[i];
        if (bh != cur) {
            widen_span(k, bh * Nk * d, Nk * d, dtype, kh);
            widen_span(v, bh * Nk * d, Nk * d, dtype, vh);
            cur = bh;
        }
        widen_span(q, (bh * Nq + r) * d, d, dtype, qr);
        dr.bh = bh;
        const uint32_t* mrow = mask_row(mask, mask_b, mask_h, H, Nq, Nk, bh, r);
        if (use_online)
            online_row(qr, kh, vh, Nk, d, causal, sc, r, key_block, st, st + (d + 2),
                       o64 + i * d, lse64 + i, max_raised ? max_raised + i : NULL, mrow);
        else
            three_step_row(qr, kh, vh, Nk, d, causal, sc, r, s, o64 + i * d, lse64 + i,
                           drop_t >= 0 ? &dr : NULL, mrow);
    }
    free(kh);
    free(vh);
    free(qr);
    free(s);
    free(st);
    return FA_ORACLE_OK;
}

int fa_ref_rows_f64(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                    int64_t Nq, int64_t Nk, int64_t d, int causal, float scale, int dtype,
                    int64_t n_sel, const int64_t* sel_bh, const int64_t* sel_row, double* o64,
                    double* lse64)
{
    return ref_rows(q, k, v, B, H, Nq, Nk, d, causal, scale, dtype, n_sel, sel_bh, sel_row, 0, 0,
                    o64, lse64, NULL, -1, 0, NULL, 1, 1);
}

int fa_ref_rows_dropout_f64(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                            int64_t Nq, int64_t Nk, int64_t d, int causal, float scale, int dtype,
                            int t, uint64_t seed, int64_t n_sel, const int64_t* sel_bh,
                            const int64_t* sel_row, double* o64, double* lse64)
{
    if (t < 0 || t > 255)
        return FA_ORACLE_EINVAL;
    return ref_rows(q, k, v, B, H, Nq, Nk, d, causal, scale, dtype, n_sel, sel_bh, sel_row, 0, 0,
                    o64, lse64, NULL, t, seed, NULL, 1, 1);
}

int fa_ref_online_f64(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                      int64_t Nq, int64_t Nk, int64_t d, int causal, float scale, int dtype,
                      int64_t n_sel, const int64_t* sel_bh, const int64_t* sel_row,
                      int64_t key_block, double* o64, double* lse64, int64_t* max_raised)
{
    return ref_rows(q, k, v, B, H, Nq, Nk, d, causal, scale, dtype, n_sel, sel_bh, sel_row, 1,
                    key_block, o64, lse64, max_raised, -1, 0, NULL, 1, 1);
}

/* The same two parts with a caller mask: mask [mask_b, mask_h, Nq, ceil(Nk / 32)] uint32
 * words, mask_b in {1, B} and mask_h in {1, H} (1 = shared by every batch / head). */
int fa_ref_rows_masked_f64(const void* q, const void* k, const void* v, const uint32_t* mask,
                           int64_t mask_b, int64_t mask_h, int64_t B, int64_t H, int64_t Nq,
                           int64_t Nk, int64_t d, int causal, float scale, int dtype,
                           int64_t n_sel, const int64_t* sel_bh, const int64_t* sel_row,
                           double* o64, double* lse64)
{
    if (!mask)
        return FA_ORACLE_EINVAL;
    return ref_rows(q, k, v, B, H, Nq, Nk, d, causal, scale, dtype, n_sel, sel_bh, sel_row, 0, 0,
                    o64, lse64, NULL, -1, 0, mask, mask_b, mask_h);
}

int fa_ref_online_masked_f64(const void* q, const void* k, const void* v, const uint32_t* mask,
                             int64_t mask_b, int64_t mask_h, int64_t B, int64_t H, int64_t Nq,
                             int64_t Nk, int64_t d, int causal, float scale, int dtype,
                             int64_t n_sel, const int64_t* sel_bh, const int64_t* sel_row,
                             int64_t key_block, double* o64, double* lse64)
{
    if (!mask)
        return FA_ORACLE_EINVAL;
    return ref_rows(q, k, v, B, H, Nq, Nk, d, causal, scale, dtype, n_sel, sel_bh, sel_row, 1,
                    key_block, o64, lse64, NULL, -1, 0, mask, mask_b, mask_h);
}

/* ------------------------------------------------------------------------- */
/* fp64 -> storage format, round to nearest, ties to even (no double rounding) */
/* ------------------------------------------------------------------------- */

/* Round x to a binary format with p significand bits (implicit bit included),
 * minimum normal exponent emin and maximum exponent emax. */
static double round_format(double x, int p, int emin, int emax)
{
    if (x != x || x == 0.0 || isinf(x))
        return x;
    int e2;
    frexp(x, &e2);      /* |x| = f * 2^e2, f in [0.5, 1): exponent of x is e2 - 1 */
    int ex = e2 - 1;
    if (ex < emin)
        ex = emin;      /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, ex - p + 1);
    double r = rint(x / quantum) * quantum; /* rint rounds half to even */
    double maxfin = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (fabs(r) > maxfin)
        return copysign(INFINITY, x);
    return r;
}

static uint16_t encode_f16(double r)
{
    /* r is exactly representable in binary16 (or +-inf / nan) */
    uint16_t sign = signbit(r) ? 0x8000 : 0;
    if (r != r)
        return 0x7e00;
    double a = fabs(r);
    if (isinf(a))
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;
    if (a < ldexp(1.0, -14))
        return sign | (uint16_t)(a / ldexp(1.0, -24)); /* subnormal */
    int e2;
    frexp(a, &e2);
    int ex = e2 - 1;
    uint16_t frac = (uint16_t)(a / ldexp(1.0, ex - 10) - 1024.0);
    return sign | (uint16_t)((ex + 15) << 10) | frac;
}

static void store_rounded(double x, int dtype, void* out, int64_t idx)
{
    if (dtype == FA_ORACLE_F32) {
        float f = (float)round_format(x, 24, -126, 127);
        memcpy((char*)out + 4 * idx, &f, 4);
    } else if (dtype == FA_ORACLE_BF16) {
        uint16_t h;
        if (x != x) {
            h = 0x7fc0;
        } else {
            float f = (float)round_format(x, 8, -126, 127); /* exact in binary32 */
            uint32_t u;
            memcpy(&u, &f, 4);
            h = (uint16_t)(u >> 16);
        }
        memcpy((char*)out + 2 * idx, &h, 2);
    } else {
        uint16_t h = encode_f16(round_format(x, 11, -14, 15));
        memcpy((char*)out + 2 * idx, &h, 2);
    }
}

int fa_oracle_round(const double* x, int64_t n, int dtype, void* out)
{
    if (!x || !out || n < 0)
        return FA_ORACLE_EINVAL;
    if (dtype != FA_ORACLE_F32 && dtype != FA_ORACLE_F16 && dtype != FA_ORACLE_BF16)
        return FA_ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        store_rounded(x[i], dtype, out, i);
    return FA_ORACLE_OK;
}

int fa_fwd_ref(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
               int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal, float scale, int dtype)
{
    int rc = check_raw(q, k, v, B, H, Nq, Nk, d, dtype);
    if (rc)
        return rc;
    if (!o || !lse)
        return FA_ORACLE_EINVAL;
    double* o64 = (double*)malloc((size_t)(Nq * d) * sizeof(double));
    double* l64 = (double*)malloc((size_t)Nq * sizeof(double));
    int64_t* bh = (int64_t*)malloc((size_t)Nq * sizeof(int64_t));
    int64_t* row = (int64_t*)malloc((size_t)Nq * sizeof(int64_t));
    if (!o64 || !l64 || !bh || !row) {
        free(o64);
        free(l64);
        free(bh);
        free(row);
        return FA_ORACLE_ENOMEM;
    }
    for (int64_t h = 0; h < B * H && rc == FA_ORACLE_OK; ++h) {
        for (int64_t r = 0; r < Nq; ++r) {
            bh[r] = h;
            row[r] = r;
        }
        rc = fa_ref_rows_f64(q, k, v, B, H, Nq, Nk, d, causal, scale, dtype, Nq, bh, row, o64,
                             l64);
        if (rc)
            break;
        for (int64_t i = 0; i < Nq * d; ++i)
            store_rounded(o64[i], dtype, o, h * Nq * d + i);
        for (int64_t r = 0; r < Nq; ++r)
            lse[h * Nq + r] = (float)l64[r];
    }
    free(o64);
    free(l64);
    free(bh);
    free(row);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Part 3: gradients of attention, the plain definition                       */
/*   [A] flash_attention_backward (course file, part 3): dV = P^T dO,          */
/*       dP = dO V^T, dS = P o (dP - D) with D_i = rowsum(dO o O),             */
/*       dQ = dS K * scale, dK = dS^T Q * scale;                               */
/*   [B] Algorithm 4 (backward pass) and its derivation: the softmax Jacobian  */
/*       diag(p) - p p^T gives dS_i = P_i o dP_i - (P_i . dP_i) P_i, and       */
/*       D_i = P_i . dP_i, which equals do_i . o_i.                            */
/* The loss whose gradients these are is sum(dO o O) for a given dO.  D is     */
/* computed here from its definition P_i . dP_i (exact in fp64, equal to       */
/* do_i . o_i up to rounding).                                                 */
/* ------------------------------------------------------------------------- */

/* P[r, :] of one query row (the softmax of the scaled, masked scores) */
static void prob_row(const double* q_row, const double* k, int64_t nk, int64_t d, int causal,
                     double scale, int64_t r, double* p, const uint32_t* mrow)
{
    double m = -INFINITY;
    for (int64_t kk = 0; kk < nk; ++kk) {
        p[kk] = score(q_row, k + kk * d, d, scale, causal, r, kk, mrow);
        if (p[kk] > m)
            m = p[kk];
    }
    if (m == -INFINITY) { /* no visible key (caller mask): P = 0 */
        for (int64_t kk = 0; kk < nk; ++kk)
            p[kk] = 0.0;
        return;
    }
    double l = 0.0;
    for (int64_t kk = 0; kk < nk; ++kk) {
        p[kk] = exp(p[kk] - m);
        l += p[kk];
    }
    for (int64_t kk = 0; kk < nk; ++kk)
        p[kk] = p[kk] / l;
}

/* dP[r, :] = (do_r V^T) o Z[r, :] and D_r = P_r . dP_r */
static double dprob_row(const double* do_row, const double* v, const double* p, int64_t nk,
                        int64_t d, double* dp, const Drop* dr, int64_t r)
{
    double D = 0.0;
    for (int64_t kk = 0; kk < nk; ++kk) {
        double acc = 0.0;
        for (int64_t t = 0; t < d; ++t)
            acc += do_row[t] * v[kk * d + t];
        dp[kk] = acc * drop_factor(dr, r, kk);
        D += p[kk] * dp[kk];
    }
    return D;
}

static int attention_bwd(const double* q, const double* k, const double* v, const double* dout,
                         int64_t nq, int64_t nk, int64_t d, int causal, double scale,
                         double* dq, double* dk, double* dv, const Drop* dr,
                         const uint32_t* mask_rows)
{
    const int64_t W = (nk + 31) / 32;
    if (!q || !k || !v || !dout || !dq || !dk || !dv || nq < 1 || nk < 1 || d < 1)
        return FA_ORACLE_EINVAL;
    double* p = (double*)malloc((size_t)nk * sizeof(double));
    double* dp = (double*)malloc((size_t)nk * sizeof(double));
    if (!p || !dp) {
        free(p);
        free(dp);
        return FA_ORACLE_ENOMEM;
    }
    for (int64_t i = 0; i < nk * d; ++i) {
        dk[i] = 0.0;
        dv[i] = 0.0;
    }
    for (int64_t r = 0; r < nq; ++r) {
        const double* q_row = q + r * d;
        const double* do_row = dout + r * d;
        prob_row(q_row, k, nk, d, causal, scale, r, p,
                 mask_rows ? mask_rows + r * W : NULL);               /* P[r, :] */
        const double D = dprob_row(do_row, v, p, nk, d, dp, dr, r); /* dP[r, :], D_r */
        for (int64_t t = 0; t < d; ++t)
            dq[r * d + t] = 0.0;
        for (int64_t kk = 0; kk < nk; ++kk) {
            const double ds = p[kk] * (dp[kk] - D); /* dS[r, kk] */
            const double pz = p[kk] * drop_factor(dr, r, kk); /* P_dropped[r, kk] */
            for (int64_t t = 0; t < d; ++t) {
                dq[r * d + t] += scale * ds * k[kk * d + t];  /* dQ = dS K * scale */
                dk[kk * d + t] += scale * ds * q_row[t];      /* dK = dS^T Q * scale */
                dv[kk * d + t] += pz * do_row[t];             /* dV = P_dropped^T dO */
            }
        }
    }
    free(p);
    free(dp);
    return FA_ORACLE_OK;
}

int fa_oracle_attention_bwd_f64(const double* q, const double* k, const double* v,
                                const double* dout, int64_t nq, int64_t nk, int64_t d,
                                int causal, double scale, double* dq, double* dk, double* dv)
{
    return attention_bwd(q, k, v, dout, nq, nk, d, causal, scale, dq, dk, dv, NULL, NULL);
}

int fa_oracle_attention_bwd_masked_f64(const double* q, const double* k, const double* v,
                                       const double* dout, const uint32_t* mask_rows, int64_t nq,
                                       int64_t nk, int64_t d, int causal, double scale,
                                       double* dq, double* dk, double* dv)
{
    if (!mask_rows)
        return FA_ORACLE_EINVAL;
    return attention_bwd(q, k, v, dout, nq, nk, d, causal, scale, dq, dk, dv, NULL, mask_rows);
}

int fa_oracle_attention_bwd_dropout_f64(const double* q, const double* k, const double* v,
                                        const double* dout, int64_t nq, int64_t nk, int64_t d,
                                        int causal, double scale, int t, uint64_t seed,
                                        int64_t bh, double* dq, double* dk, double* dv)
{
    Drop dr;
    if (bh < 0 || make_drop(&dr, t, seed, bh))
        return FA_ORACLE_EINVAL;
    return attention_bwd(q, k, v, dout, nq, nk, d, causal, scale, dq, dk, dv, &dr, NULL);
}

/* raw-buffer gradients ---------------------------------------------------- */

static int check_bwd_raw(const void* q, const void* k, const void* v, const void* dout,
                         int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int dtype)
{
    if (!dout)
        return FA_ORACLE_EINVAL;
    return check_raw(q, k, v, B, H, Nq, Nk, d, dtype);
}

static int bwd_head(const void* q, const void* k, const void* v, const void* dout, int64_t B,
                    int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                    int dtype, int64_t bh, double* dq64, double* dk64, double* dv64,
                    const Drop* dr, const uint32_t* mask, int64_t mask_b, int64_t mask_h)
{
    int rc = check_bwd_raw(q, k, v, dout, B, H, Nq, Nk, d, dtype);
    if (rc)
        return rc;
    if (check_mask(mask, mask_b, mask_h, B, H))
        return FA_ORACLE_EINVAL;
    if (bh < 0 || bh >= B * H || !dq64 || !dk64 || !dv64)
        return FA_ORACLE_EINVAL;
    double* buf = (double*)malloc((size_t)(2 * Nq * d + 2 * Nk * d) * sizeof(double));
    if (!buf)
        return FA_ORACLE_ENOMEM;
    double *qh = buf, *doh = buf + Nq * d, *kh = doh + Nq * d, *vh = kh + Nk * d;
    widen_span(q, bh * Nq * d, Nq * d, dtype, qh);
    widen_span(dout, bh * Nq * d, Nq * d, dtype, doh);
    widen_span(k, bh * Nk * d, Nk * d, dtype, kh);
    widen_span(v, bh * Nk * d, Nk * d, dtype, vh);
    rc = attention_bwd(qh, kh, vh, doh, Nq, Nk, d, causal, (double)scale, dq64, dk64, dv64, dr,
                       mask_row(mask, mask_b, mask_h, H, Nq, Nk, bh, 0));
    free(buf);
    return rc;
}

/* One head bh of raw [B,H,N,d] buffers: every row of dQ and every key of dK, dV. */
int fa_ref_bwd_head_f64(const void* q, const void* k, const void* v, const void* dout,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                        float scale, int dtype, int64_t bh, double* dq64, double* dk64,
                        double* dv64)
{
    return bwd_head(q, k, v, dout, B, H, Nq, Nk, d, causal, scale, dtype, bh, dq64, dk64, dv64,
                    NULL, NULL, 1, 1);
}

/* The same with a caller mask ([mask_b, mask_h, Nq, ceil(Nk / 32)] words, as
 * fa_ref_rows_masked_f64). */
int fa_ref_bwd_head_masked_f64(const void* q, const void* k, const void* v, const void* dout,
                               const uint32_t* mask, int64_t mask_b, int64_t mask_h, int64_t B,
                               int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                               float scale, int dtype, int64_t bh, double* dq64, double* dk64,
                               double* dv64)
{
    if (!mask)
        return FA_ORACLE_EINVAL;
    return bwd_head(q, k, v, dout, B, H, Nq, Nk, d, causal, scale, dtype, bh, dq64, dk64, dv64,
                    NULL, mask, mask_b, mask_h);
}

/* The same with dropout (threshold t, seed) on P. */
int fa_ref_bwd_head_dropout_f64(const void* q, const void* k, const void* v, const void* dout,
                                int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                int causal, float scale, int dtype, int t, uint64_t seed,
                                int64_t bh, double* dq64, double* dk64, double* dv64)
{
    Drop dr;
    if (make_drop(&dr, t, seed, bh))
        return FA_ORACLE_EINVAL;
    return bwd_head(q, k, v, dout, B, H, Nq, Nk, d, causal, scale, dtype, bh, dq64, dk64, dv64,
                    &dr, NULL, 1, 1);
}

/* dQ of selected query rows (sel_bh[i], sel_row[i]) -> dq64[i * d .. +d] */
int fa_ref_bwd_dq_rows_f64(const void* q, const void* k, const void* v, const void* dout,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                           float scale, int dtype, int64_t n_sel, const int64_t* sel_bh,
                           const int64_t* sel_row, double* dq64)
{
    int rc = check_bwd_raw(q, k, v, dout, B, H, Nq, Nk, d, dtype);
    if (rc)
        return rc;
    if (n_sel < 0 || (n_sel > 0 && (!sel_bh || !sel_row || !dq64)))
        return FA_ORACLE_EINVAL;
    for (int64_t i = 0; i < n_sel; ++i)
        if (sel_bh[i] < 0 || sel_bh[i] >= B * H || sel_row[i] < 0 || sel_row[i] >= Nq)
            return FA_ORACLE_EINVAL;
    double* buf = (double*)malloc((size_t)(2 * Nk * d + 2 * d + 2 * Nk) * sizeof(double));
    if (!buf)
        return FA_ORACLE_ENOMEM;
    double *kh = buf, *vh = kh + Nk * d, *qr = vh + Nk * d, *dor = qr + d, *p = dor + d,
           *dp = p + Nk;
    const double sc = (double)scale;
    int64_t cur = -1;
    for (int64_t i = 0; i < n_sel; ++i) {
        const int64_t bh = sel_bh[i], r = sel_row[i];
        if (bh != cur) {
            widen_span(k, bh * Nk * d, Nk * d, dtype, kh);
            widen_span(v, bh * Nk * d, Nk * d, dtype, vh);
            cur = bh;
        }
        widen_span(q, (bh * Nq + r) * d, d, dtype, qr);
        widen_span(dout, (bh * Nq + r) * d, d, dtype, dor);
        prob_row(qr, kh, Nk, d, causal, sc, r, p, NULL);
        const double D = dprob_row(dor, vh, p, Nk, d, dp, NULL, r);
        double* out = dq64 + i * d;
        for (int64_t t = 0; t < d; ++t)
            out[t] = 0.0;
        for (int64_t kk = 0; kk < Nk; ++kk) {
            const double ds = p[kk] * (dp[kk] - D);
            for (int64_t t = 0; t < d; ++t)
                out[t] += sc * ds * kh[kk * d + t];
        }
    }
    free(buf);
    return FA_ORACLE_OK;
}

/* Per-row statistics of selected rows: lse64[i] = log-sum-exp of the scaled, masked
 * scores of row (sel_bh[i], sel_row[i]) and D64[i] = P_r . dP_r. */
int fa_ref_bwd_rowstats_f64(const void* q, const void* k, const void* v, const void* dout,
                            int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                            float scale, int dtype, int64_t n_sel, const int64_t* sel_bh,
                            const int64_t* sel_row, double* lse64, double* D64)
{
    int rc = check_bwd_raw(q, k, v, dout, B, H, Nq, Nk, d, dtype);
    if (rc)
        return rc;
    if (n_sel < 0 || (n_sel > 0 && (!sel_bh || !sel_row || !lse64 || !D64)))
        return FA_ORACLE_EINVAL;
    for (int64_t i = 0; i < n_sel; ++i)
        if (sel_bh[i] < 0 || sel_bh[i] >= B * H || sel_row[i] < 0 || sel_row[i] >= Nq)
            return FA_ORACLE_EINVAL;
    double* buf = (double*)malloc((size_t)(2 * Nk * d + 2 * d + 2 * Nk + d) * sizeof(double));
    if (!buf)
        return FA_ORACLE_ENOMEM;
    double *kh = buf, *vh = kh + Nk * d, *qr = vh + Nk * d, *dor = qr + d, *p = dor + d,
           *dp = p + Nk, *o_row = dp + Nk;
    const double sc = (double)scale;
    int64_t cur = -1;
    for (int64_t i = 0; i < n_sel; ++i) {
        const int64_t bh = sel_bh[i], r = sel_row[i];
        if (bh != cur) {
            widen_span(k, bh * Nk * d, Nk * d, dtype, kh);
            widen_span(v, bh * Nk * d, Nk * d, dtype, vh);
            cur = bh;
        }
        widen_span(q, (bh * Nq + r) * d, d, dtype, qr);
        widen_span(dout, (bh * Nq + r) * d, d, dtype, dor);
        three_step_row(qr, kh, vh, Nk, d, causal, sc, r, p, o_row, lse64 + i, NULL, NULL);
        prob_row(qr, kh, Nk, d, causal, sc, r, p, NULL);
        D64[i] = dprob_row(dor, vh, p, Nk, d, dp, NULL, r);
    }
    free(buf);
    return FA_ORACLE_OK;
}

/* dK and dV of selected keys (sel_bh[i], sel_key[i]), given every row's statistics
 * of the heads involved (lse64_all and D64_all, [B*H*Nq], from
 * fa_ref_bwd_rowstats_f64): P[r, j] = exp(S[r, j] - lse_r),
 * dv_j = sum_r P[r, j] do_r, dk_j = scale * sum_r P[r, j] (dP[r, j] - D_r) q_r. */
int fa_ref_bwd_dkv_keys_f64(const void* q, const void* k, const void* v, const void* dout,
                            int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                            float scale, int dtype, const double* lse64_all,
                            const double* D64_all, int64_t n_sel, const int64_t* sel_bh,
                            const int64_t* sel_key, double* dk64, double* dv64)
{
    int rc = check_bwd_raw(q, k, v, dout, B, H, Nq, Nk, d, dtype);
    if (rc)
        return rc;
    if (!lse64_all || !D64_all || n_sel < 0 ||
        (n_sel > 0 && (!sel_bh || !sel_key || !dk64 || !dv64)))
        return FA_ORACLE_EINVAL;
    for (int64_t i = 0; i < n_sel; ++i)
        if (sel_bh[i] < 0 || sel_bh[i] >= B * H || sel_key[i] < 0 || sel_key[i] >= Nk)
            return FA_ORACLE_EINVAL;
    double* buf = (double*)malloc((size_t)(2 * Nq * d + 2 * d) * sizeof(double));
    if (!buf)
        return FA_ORACLE_ENOMEM;
    double *qh = buf, *doh = qh + Nq * d, *kr = doh + Nq * d, *vr = kr + d;
    const double sc = (double)scale;
    int64_t cur = -1;
    for (int64_t i = 0; i < n_sel; ++i) {
        const int64_t bh = sel_bh[i], j = sel_key[i];
        if (bh != cur) {
            widen_span(q, bh * Nq * d, Nq * d, dtype, qh);
            widen_span(dout, bh * Nq * d, Nq * d, dtype, doh);
            cur = bh;
        }
        widen_span(k, (bh * Nk + j) * d, d, dtype, kr);
        widen_span(v, (bh * Nk + j) * d, d, dtype, vr);
        double* dkj = dk64 + i * d;
        double* dvj = dv64 + i * d;
        for (int64_t t = 0; t < d; ++t) {
            dkj[t] = 0.0;
            dvj[t] = 0.0;
        }
        for (int64_t r = 0; r < Nq; ++r) {
            const double s = score(qh + r * d, kr, d, sc, causal, r, j, NULL);
            if (s == -INFINITY)
                continue; /* masked: P[r, j] = 0 */
            const double p = exp(s - lse64_all[bh * Nq + r]);
            double dp = 0.0;
            for (int64_t t = 0; t < d; ++t)
                dp += doh[r * d + t] * vr[t];
            const double ds = p * (dp - D64_all[bh * Nq + r]);
            for (int64_t t = 0; t < d; ++t) {
                dvj[t] += p * doh[r * d + t];
                dkj[t] += sc * ds * qh[r * d + t];
            }
        }
    }
    free(buf);
    return FA_ORACLE_OK;
}

/* Host counterpart of the GPU backward: dq, dk, dv of every head, rounded to dtype. */
int fa_bwd_ref(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
               void* dv, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
               float scale, int dtype)
{
    int rc = check_bwd_raw(q, k, v, dout, B, H, Nq, Nk, d, dtype);
    if (rc)
        return rc;
    if (!dq || !dk || !dv)
        return FA_ORACLE_EINVAL;
    double* g = (double*)malloc((size_t)(Nq * d + 2 * Nk * d) * sizeof(double));
    if (!g)
        return FA_ORACLE_ENOMEM;
    for (int64_t bh = 0; bh < B * H && rc == FA_ORACLE_OK; ++bh) {
        rc = fa_ref_bwd_head_f64(q, k, v, dout, B, H, Nq, Nk, d, causal, scale, dtype, bh, g,
                                 g + Nq * d, g + Nq * d + Nk * d);
        if (rc)
            break;
        for (int64_t i = 0; i < Nq * d; ++i)
            store_rounded(g[i], dtype, dq, bh * Nq * d + i);
        for (int64_t i = 0; i < Nk * d; ++i) {
            store_rounded(g[Nq * d + i], dtype, dk, bh * Nk * d + i);
            store_rounded(g[Nq * d + Nk * d + i], dtype, dv, bh * Nk * d + i);
        }
    }
    free(g);
    return rc;
}
