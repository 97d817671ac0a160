/* Sanitizer driver for the oracle (oracle/fa_oracle.c): every exported function on small
 * inputs of each storage type, masks with a row that sees no key, dropout, the gradients
 * and the argument checks.  Built with -fsanitize=address,undefined and halting on the
 * first finding; prints "ok" when every call returned what it should. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/fa_oracle.h"

static uint32_t lcg = 12345u;
static uint32_t next_u32(void)
{
    lcg = lcg * 1664525u + 1013904223u;
    return lcg;
}
static double rnd(void) { return ((double)(next_u32() >> 8) / 16777216.0) * 2.0 - 1.0; }

static double* fill(int64_t n)
{
    double* p = malloc(sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; ++i)
        p[i] = rnd();
    return p;
}

enum { NQ = 37, NK = 70, D = 16, W = (NK + 31) / 32, B = 2, H = 3, BH = B * H };

int main(void)
{
    int rc = 0;
    /* one-dimensional online softmax and the merge */
    double *x = fill(50), *y = fill(50), st[4][8];
    rc |= fa_oracle_softmax_online(x, 50, 7, y, st[0], st[1], st[2], st[3]);
    double a3[3] = {0.5, 2.0, 1.0}, b3[3] = {1.5, 1.0, -1.0}, m3[3];
    rc |= fa_oracle_merge(1, a3, b3, m3);

    /* fp64 per-head parts */
    double *q = fill(NQ * D), *k = fill(NK * D), *v = fill(NK * D), *dout = fill(NQ * D);
    double *o = malloc(sizeof(double) * NQ * D), *lse = malloc(sizeof(double) * NQ);
    double *dq = malloc(sizeof(double) * NQ * D), *dk = malloc(sizeof(double) * NK * D);
    double* dv = malloc(sizeof(double) * NK * D);
    uint32_t* mask = malloc(sizeof(uint32_t) * NQ * W);
    int64_t rows[NQ], raised[NQ];
    for (int i = 0; i < NQ; ++i)
        rows[i] = i;
    for (int i = 0; i < NQ * W; ++i)
        mask[i] = next_u32();
    memset(mask + 3 * W, 0, sizeof(uint32_t) * W); /* a row with no visible key */
    for (int causal = 0; causal < 2; ++causal) {
        rc |= fa_oracle_attention_f64(q, k, v, NQ, NK, D, causal, 0.25, NQ, rows, o, lse);
        rc |= fa_oracle_online_f64(q, k, v, NQ, NK, D, causal, 0.25, 7, NQ, rows, o, lse, raised);
        rc |= fa_oracle_attention_bwd_f64(q, k, v, dout, NQ, NK, D, causal, 0.25, dq, dk, dv);
        rc |= fa_oracle_attention_masked_f64(q, k, v, mask, NQ, NK, D, causal, 0.25, NQ, rows, o,
                                             lse);
        rc |= fa_oracle_online_masked_f64(q, k, v, mask, NQ, NK, D, causal, 0.25, 5, NQ, rows, o,
                                          lse);
        rc |= fa_oracle_attention_bwd_masked_f64(q, k, v, dout, mask, NQ, NK, D, causal, 0.25, dq,
                                                 dk, dv);
        rc |= fa_oracle_attention_dropout_f64(q, k, v, NQ, NK, D, causal, 0.25, 40, 7, 1, NQ, rows,
                                              o, lse);
        rc |= fa_oracle_attention_bwd_dropout_f64(q, k, v, dout, NQ, NK, D, causal, 0.25, 40, 7, 1,
                                                  dq, dk, dv);
    }
    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, ph[4];
    rc |= fa_oracle_philox4x32_10(ctr, key, ph);
    uint8_t* keep = malloc(NQ * NK);
    rc |= fa_oracle_dropout_keep(99, 128, 2, NQ, NK, keep);

    /* raw buffers of each storage type, [B, H, N, D], rounded from fp64 by the oracle */
    double *q64 = fill(BH * NQ * D), *k64 = fill(BH * NK * D), *v64 = fill(BH * NK * D);
    double* d64 = fill(BH * NQ * D);
    void *qr = malloc(4 * BH * NQ * D), *kr = malloc(4 * BH * NK * D), *vr = malloc(4 * BH * NK * D);
    void *dr = malloc(4 * BH * NQ * D), *orw = malloc(4 * BH * NQ * D);
    void *dqr = malloc(4 * BH * NQ * D), *dkr = malloc(4 * BH * NK * D), *dvr = malloc(4 * BH * NK * D);
    float* lf = malloc(sizeof(float) * BH * NQ);
    uint32_t* mask_bh = malloc(sizeof(uint32_t) * BH * NQ * W);
    for (int i = 0; i < BH * NQ * W; ++i)
        mask_bh[i] = next_u32();
    memset(mask_bh + 5 * W, 0, sizeof(uint32_t) * W);
    int64_t sel_bh[BH * NQ], sel_row[BH * NQ], sel_key[NK], sel_kbh[NK];
    for (int i = 0; i < BH * NQ; ++i) {
        sel_bh[i] = i / NQ;
        sel_row[i] = i % NQ;
    }
    for (int i = 0; i < NK; ++i) {
        sel_key[i] = i;
        sel_kbh[i] = 4;
    }
    double *o64 = malloc(sizeof(double) * BH * NQ * D), *l64 = malloc(sizeof(double) * BH * NQ);
    double* D64 = malloc(sizeof(double) * BH * NQ);
    double *gq = malloc(sizeof(double) * NQ * D), *gk = malloc(sizeof(double) * NK * D);
    double* gv = malloc(sizeof(double) * NK * D);
    double *gq_all = malloc(sizeof(double) * BH * NQ * D), *gk_all = malloc(sizeof(double) * NK * D);
    double* gv_all = malloc(sizeof(double) * NK * D);
    for (int dt = 0; dt < 3; ++dt) {
        rc |= fa_oracle_round(q64, BH * NQ * D, dt, qr);
        rc |= fa_oracle_round(k64, BH * NK * D, dt, kr);
        rc |= fa_oracle_round(v64, BH * NK * D, dt, vr);
        rc |= fa_oracle_round(d64, BH * NQ * D, dt, dr);
        for (int causal = 0; causal < 2; ++causal) {
            rc |= fa_ref_rows_f64(qr, kr, vr, B, H, NQ, NK, D, causal, 0.25f, dt, BH * NQ, sel_bh,
                                  sel_row, o64, l64);
            rc |= fa_ref_online_f64(qr, kr, vr, B, H, NQ, NK, D, causal, 0.25f, dt, BH * NQ,
                                    sel_bh, sel_row, 9, o64, l64, NULL);
            rc |= fa_ref_rows_masked_f64(qr, kr, vr, mask_bh, B, H, B, H, NQ, NK, D, causal, 0.25f,
                                         dt, BH * NQ, sel_bh, sel_row, o64, l64);
            rc |= fa_ref_rows_masked_f64(qr, kr, vr, mask_bh, 1, 1, B, H, NQ, NK, D, causal, 0.25f,
                                         dt, BH * NQ, sel_bh, sel_row, o64, l64);
            rc |= fa_ref_online_masked_f64(qr, kr, vr, mask_bh, 1, H, B, H, NQ, NK, D, causal,
                                           0.25f, dt, BH * NQ, sel_bh, sel_row, 9, o64, l64);
            rc |= fa_ref_rows_dropout_f64(qr, kr, vr, B, H, NQ, NK, D, causal, 0.25f, dt, 60, 3,
                                          BH * NQ, sel_bh, sel_row, o64, l64);
            rc |= fa_ref_bwd_head_f64(qr, kr, vr, dr, B, H, NQ, NK, D, causal, 0.25f, dt, 5, gq,
                                      gk, gv);
            rc |= fa_ref_bwd_head_masked_f64(qr, kr, vr, dr, mask_bh, B, H, B, H, NQ, NK, D,
                                             causal, 0.25f, dt, 0, gq, gk, gv);
            rc |= fa_ref_bwd_head_dropout_f64(qr, kr, vr, dr, B, H, NQ, NK, D, causal, 0.25f, dt,
                                              90, 11, 2, gq, gk, gv);
            rc |= fa_ref_bwd_dq_rows_f64(qr, kr, vr, dr, B, H, NQ, NK, D, causal, 0.25f, dt,
                                         BH * NQ, sel_bh, sel_row, gq_all);
            rc |= fa_ref_bwd_rowstats_f64(qr, kr, vr, dr, B, H, NQ, NK, D, causal, 0.25f, dt,
                                          BH * NQ, sel_bh, sel_row, l64, D64);
            rc |= fa_ref_bwd_dkv_keys_f64(qr, kr, vr, dr, B, H, NQ, NK, D, causal, 0.25f, dt, l64,
                                          D64, NK, sel_kbh, sel_key, gk_all, gv_all);
            rc |= fa_fwd_ref(qr, kr, vr, orw, lf, B, H, NQ, NK, D, causal, 0.25f, dt);
            rc |= fa_bwd_ref(qr, kr, vr, dr, dqr, dkr, dvr, B, H, NQ, NK, D, causal, 0.25f, dt);
        }
    }
    /* argument checks: each must be refused with FA_ORACLE_EINVAL, not crash */
    int refused = 0;
    refused += fa_oracle_attention_f64(NULL, k, v, NQ, NK, D, 0, 0.25, NQ, rows, o, lse) ==
               FA_ORACLE_EINVAL;
    refused += fa_ref_rows_f64(qr, kr, vr, B, H, NQ, NK, D, 0, 0.25f, 7, 1, sel_bh, sel_row, o64,
                               l64) == FA_ORACLE_EINVAL;
    refused += fa_ref_rows_masked_f64(qr, kr, vr, mask_bh, 3, 1, B, H, NQ, NK, D, 0, 0.25f, 0, 1,
                                      sel_bh, sel_row, o64, l64) == FA_ORACLE_EINVAL;
    refused += fa_ref_rows_masked_f64(qr, kr, vr, NULL, 1, 1, B, H, NQ, NK, D, 0, 0.25f, 0, 1,
                                      sel_bh, sel_row, o64, l64) == FA_ORACLE_EINVAL;
    int64_t bad_row = NQ;
    refused += fa_ref_rows_f64(qr, kr, vr, B, H, NQ, NK, D, 0, 0.25f, 0, 1, sel_bh, &bad_row, o64,
                               l64) == FA_ORACLE_EINVAL;
    refused += fa_oracle_dropout_keep(1, 256, 0, NQ, NK, keep) == FA_ORACLE_EINVAL;
    if (rc != 0 || refused != 6) {
        printf("failed: rc=%d refused=%d of 6\n", rc, refused);
        return 1;
    }
    free(x); free(y); free(q); free(k); free(v); free(dout); free(o); free(lse); free(dq);
    free(dk); free(dv); free(mask); free(keep); free(q64); free(k64); free(v64); free(d64);
    free(qr); free(kr); free(vr); free(dr); free(orw); free(dqr); free(dkr); free(dvr); free(lf);
    free(mask_bh); free(o64); free(l64); free(D64); free(gq); free(gk); free(gv); free(gq_all);
    free(gk_all); free(gv_all);
    printf("ok\n");
    return 0;
}
