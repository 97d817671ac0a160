/*
 * fa_oracle.h — C-ABI of the fp64 CPU oracle (test infrastructure only).
 *
 * The oracle is a plain, slow, obviously-correct host implementation of what the
 * fused attention forward pass (and its gradients) compute.  It exists to check the GPU library
 * (fa.h) and is built into its own shared library, libfa_oracle.so, from
 * oracle/fa_oracle.c.  The GPU library never links it, and it shares no code,
 * header or table with the GPU library: the dtype codes below are restated here
 * with the same numeric values as fa.h because both describe the same buffers.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * Definitions followed (pages as cited in the sources):
 *   - standard three-step attention: S = scale * Q K^T, P = row-softmax(S), O = P V
 *     ("05_flash_attention.py" course file, function standard_attention;
 *      "Flash Attention" blog page, section "Why Flash Attention" and Algorithm 2
 *      for the scale tau and the mask);
 *   - causal visibility: key k is visible to query q iff k <= q, indices 0-based,
 *     aligned at the top-left corner (course file, standard_attention's triu(1) mask);
 *   - row logsumexp L = m + ln(l), natural log (course file, flash_attention_forward
 *     and demo_online_softmax);
 *   - online softmax and the (+) merge on (m, d) and (m, d, o~)
 *     ("Flash Attention" blog page, sections "Online Softmax" and parallelisation);
 *   - gradients of the loss sum(dO o O): dV = P^T dO, dP = dO V^T,
 *     dS = P o (dP - D) with D_r = P_r . dP_r (= do_r . o_r), dQ = scale dS K,
 *     dK = scale dS^T Q (course file, flash_attention_backward; blog page,
 *     Algorithm 4 and the softmax-Jacobian derivation after it).
 *
 * Conventions common to every function:
 *   - all pointers are HOST pointers; the caller owns every buffer;
 *   - the functions are synchronous, re-entrant and thread-safe (they keep no
 *     global state; scratch memory is malloc'd per call and freed before return);
 *   - return value: 0 on success, FA_ORACLE_EINVAL (1) on an invalid argument,
 *     FA_ORACLE_ENOMEM (4) if a scratch allocation fails; outputs are then untouched
 *     or partially written;
 *   - tensors are contiguous: q and o are [B,H,Nq,d], k and v are [B,H,Nk,d],
 *     lse is [B,H,Nq], d fastest;
 *   - arithmetic is IEEE fp64 with plain left-to-right summation.
 */
#ifndef FA_ORACLE_H
#define FA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of q, k, v (and o for fa_fwd_ref); same codes as fa.h */
enum { FA_ORACLE_F32 = 0, FA_ORACLE_F16 = 1, FA_ORACLE_BF16 = 2 };

enum { FA_ORACLE_OK = 0, FA_ORACLE_EINVAL = 1, FA_ORACLE_ENOMEM = 4 };

/*
 * One-dimensional online softmax over x[0..n) read in blocks of `block` values
 * (course file, online_softmax_stats; blog page "Online Softmax").
 * Per block b (nb = ceil(n/block) blocks), after reading it:
 *   run_m[b]   running maximum m_b;
 *   run_l[b]   running sum l_b = sum_{k read so far} exp(x_k - m_b);
 *   carried[b] the previous sum carried over, l_{b-1} * exp(m_{b-1} - m_b) (0 for b = 0);
 *   fresh[b]   the new block's own sum relative to the new maximum, sum exp(x_k - m_b).
 * y[0..n) receives the final softmax exp(x_i - m_last) / l_last (second pass).
 * Any trace pointer may be NULL.  n >= 1, block >= 1.  -inf entries are allowed as
 * long as x holds at least one finite value.
 */
int fa_oracle_softmax_online(const double* x, int64_t n, int64_t block, double* y,
                             double* run_m, double* run_l, double* carried, double* fresh);

/*
 * The (+) merge of two online-softmax states (blog page, the extended operator on
 * (m, d, o~)).  A state is packed as [m, d, o~_0 .. o~_{dim-1}] (dim+2 doubles).
 * out may alias a or b.  The empty state (m = -inf, d = 0, o~ = 0) is the identity.
 */
int fa_oracle_merge(int64_t dim, const double* a, const double* b, double* out);

/*
 * Part 1 — standard three-step attention for selected query rows of ONE head,
 * on fp64 inputs: q [nq,d], k [nk,d], v [nk,d].  For each i < n_rows, row r = rows[i]:
 * materialise s_k = scale * <q_r, k_k> for every key (-inf when causal and k > r),
 * safe softmax (max, exp, sum, normalise), then o = sum_k p_k v_k.
 * Writes o[i*d .. i*d+d) and lse[i] = m + ln(l).
 */
int fa_oracle_attention_f64(const double* q, const double* k, const double* v,
                            int64_t nq, int64_t nk, int64_t d, int causal, double scale,
                            int64_t n_rows, const int64_t* rows, double* o, double* lse);

/*
 * Part 2 — scalar online (m, d, o~) accumulator, same contract as part 1.
 * key_block <= 0: keys are consumed one at a time (blog page recurrence);
 * key_block  > 0: each contiguous block of key_block keys is first reduced to its own
 * state by the scalar recurrence, then folded into the running state with the (+) merge.
 * Masked keys are skipped.  If max_raised is not NULL, max_raised[i] counts how often
 * the running maximum of row i increased after the first visible key.
 */
int fa_oracle_online_f64(const double* q, const double* k, const double* v,
                         int64_t nq, int64_t nk, int64_t d, int causal, double scale,
                         int64_t key_block, int64_t n_rows, const int64_t* rows,
                         double* o, double* lse, int64_t* max_raised);

/*
 * Part 1 on the raw input buffers the GPU receives: q, k, v hold `dtype` elements
 * (bf16/fp16 bit patterns or fp32), widened exactly to fp64.  The n_sel selected rows
 * are (sel_bh[i], sel_row[i]) with sel_bh = b*H + h.  Outputs: o64 [n_sel, d] and
 * lse64 [n_sel].  `scale` is the fp32 value passed to the GPU, widened exactly.
 * Rows belonging to the same head should be adjacent (K and V of a head are widened
 * once per run of equal sel_bh).  Requires B, H, Nq, Nk, d >= 1.
 */
int fa_ref_rows_f64(const void* q, const void* k, const void* v,
                    int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                    int causal, float scale, int dtype,
                    int64_t n_sel, const int64_t* sel_bh, const int64_t* sel_row,
                    double* o64, double* lse64);

/* Part 2 on raw input buffers; same contract as fa_ref_rows_f64 plus key_block. */
int fa_ref_online_f64(const void* q, const void* k, const void* v,
                      int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                      int causal, float scale, int dtype,
                      int64_t n_sel, const int64_t* sel_bh, const int64_t* sel_row,
                      int64_t key_block, double* o64, double* lse64, int64_t* max_raised);

/*
 * Whole-tensor host counterpart of fa_fwd: every row through part 1, then o is
 * rounded from fp64 to `dtype` with round-to-nearest-even (directly, no double
 * rounding) and lse to fp32.  Synchronous; o and lse are host buffers.
 */
int fa_fwd_ref(const void* q, const void* k, const void* v, void* o, float* lse,
               int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
               int causal, float scale, int dtype);

/* fp64 -> dtype rounding used by fa_fwd_ref (round to nearest, ties to even),
 * exposed so that it can be pinned against independent conversions. */
int fa_oracle_round(const double* x, int64_t n, int dtype, void* out);

/*
 * Part 3: gradients, plain definition, one head of fp64 inputs (row-major
 * q, dout [nq, d], k, v [nk, d]).  Writes dq [nq, d], dk, dv [nk, d].  Every row
 * materialises P_r and dP_r = do_r V^T, takes D_r = P_r . dP_r and
 * dS_r = P_r o (dP_r - D_r), and accumulates dq_r = scale dS_r K,
 * dk += scale dS_r^T q_r, dv += P_r^T do_r.
 */
int fa_oracle_attention_bwd_f64(const double* q, const double* k, const double* v,
                                const double* dout, int64_t nq, int64_t nk, int64_t d,
                                int causal, double scale, double* dq, double* dk, double* dv);

/* Part 3 on head bh of raw [B,H,N,d] buffers of `dtype` (dout like q): fp64 dq64
 * [Nq, d], dk64 and dv64 [Nk, d]. */
int fa_ref_bwd_head_f64(const void* q, const void* k, const void* v, const void* dout,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                        float scale, int dtype, int64_t bh, double* dq64, double* dk64,
                        double* dv64);

/* dQ of selected rows (sel_bh[i], sel_row[i]) of raw buffers -> dq64 [n_sel, d]. */
int fa_ref_bwd_dq_rows_f64(const void* q, const void* k, const void* v, const void* dout,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                           float scale, int dtype, int64_t n_sel, const int64_t* sel_bh,
                           const int64_t* sel_row, double* dq64);

/* Row statistics of selected rows: lse64[i] (as part 1) and D64[i] = P_r . dP_r. */
int fa_ref_bwd_rowstats_f64(const void* q, const void* k, const void* v, const void* dout,
                            int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                            float scale, int dtype, int64_t n_sel, const int64_t* sel_bh,
                            const int64_t* sel_row, double* lse64, double* D64);

/* dK and dV of selected keys (sel_bh[i], sel_key[i]) -> dk64, dv64 [n_sel, d], given
 * the row statistics of every row of the heads involved (lse64_all, D64_all indexed
 * [bh * Nq + r]): P[r, j] = exp(S[r, j] - lse_r), dv_j = sum_r P[r, j] do_r,
 * dk_j = scale sum_r P[r, j] (dP[r, j] - D_r) q_r. */
int fa_ref_bwd_dkv_keys_f64(const void* q, const void* k, const void* v, const void* dout,
                            int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                            float scale, int dtype, const double* lse64_all,
                            const double* D64_all, int64_t n_sel, const int64_t* sel_bh,
                            const int64_t* sel_key, double* dk64, double* dv64);

/*
 * Dropout on P (blog page, Algorithm 2 and Algorithm 4, whose random numbers the
 * pages leave open).  Reading: Philox4x32-10 (Salmon et al., SC'11) with key
 * (seed low, seed high) and counter (k/4, q/4, bh, 0); element (q, k) takes output
 * byte 4(q%4) + k%4 (byte b of word w = bits 8b.. of w, index 4w + b) and is dropped
 * iff that byte is below t (0 <= t <= 255); kept elements are scaled by
 * 256 / (256 - t).  L is unchanged (the softmax's), O = (P o Z) V, and in the
 * gradients dV = (P o Z)^T dO and dP = (dO V^T) o Z.
 */
int fa_oracle_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out);
/* keep[q * nk + k] = 1 where element (q, k) of head bh is kept, else 0 */
int fa_oracle_dropout_keep(uint64_t seed, int t, int64_t bh, int64_t nq, int64_t nk,
                           uint8_t* keep);
/* Part 1 with dropout on P (head index bh selects the random numbers). */
int fa_oracle_attention_dropout_f64(const double* q, const double* k, const double* v,
                                    int64_t nq, int64_t nk, int64_t d, int causal, double scale,
                                    int t, uint64_t seed, int64_t bh, int64_t n_rows,
                                    const int64_t* rows, double* o, double* lse);
/* Part 3 with dropout on P. */
int fa_oracle_attention_bwd_dropout_f64(const double* q, const double* k, const double* v,
                                        const double* dout, int64_t nq, int64_t nk, int64_t d,
                                        int causal, double scale, int t, uint64_t seed,
                                        int64_t bh, double* dq, double* dk, double* dv);
/* Raw-buffer counterparts of the two above (selected rows; one head). */
int fa_ref_rows_dropout_f64(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                            int64_t Nq, int64_t Nk, int64_t d, int causal, float scale, int dtype,
                            int t, uint64_t seed, int64_t n_sel, const int64_t* sel_bh,
                            const int64_t* sel_row, double* o64, double* lse64);
int fa_ref_bwd_head_dropout_f64(const void* q, const void* k, const void* v, const void* dout,
                                int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                int causal, float scale, int dtype, int t, uint64_t seed,
                                int64_t bh, double* dq64, double* dk64, double* dv64);

/*
 * Part 5: caller masks (blog page "Flash Attention", Algorithm 2: S_masked = mask(S),
 * P = softmax(S_masked); Algorithm 4 recomputes P from mask(S)).  Reading: mask(S)
 * sets S[q, k] to -inf where the caller's boolean mask is false (after the causal rule
 * when causal = 1: both must allow the key).  A query row's mask is bit-packed: key k
 * in bit k % 32 of 32-bit word k / 32, set = visible; one row holds W = ceil(Nk / 32)
 * words.  A row with no visible key has no softmax; the reading taken: O = 0 and
 * L = -inf (the identity of the (+) merge), P = 0 in the gradients.
 *
 * mask_rows of the double-array forms: [nq, W] words for the one head.  mask of the
 * raw-buffer forms: [mask_b, mask_h, Nq, W] words with mask_b in {1, B} and mask_h in
 * {1, H} (an extent of 1 is shared by every batch / head).
 */
int fa_oracle_attention_masked_f64(const double* q, const double* k, const double* v,
                                   const uint32_t* mask_rows, int64_t nq, int64_t nk, int64_t d,
                                   int causal, double scale, int64_t n_rows, const int64_t* rows,
                                   double* o, double* lse);
int fa_oracle_online_masked_f64(const double* q, const double* k, const double* v,
                                const uint32_t* mask_rows, int64_t nq, int64_t nk, int64_t d,
                                int causal, double scale, int64_t key_block, int64_t n_rows,
                                const int64_t* rows, double* o, double* lse);
int fa_oracle_attention_bwd_masked_f64(const double* q, const double* k, const double* v,
                                       const double* dout, const uint32_t* mask_rows, int64_t nq,
                                       int64_t nk, int64_t d, int causal, double scale,
                                       double* dq, double* dk, double* dv);
int fa_ref_rows_masked_f64(const void* q, const void* k, const void* v, const uint32_t* mask,
                           int64_t mask_b, int64_t mask_h, int64_t B, int64_t H, int64_t Nq,
                           int64_t Nk, int64_t d, int causal, float scale, int dtype,
                           int64_t n_sel, const int64_t* sel_bh, const int64_t* sel_row,
                           double* o64, double* lse64);
int fa_ref_online_masked_f64(const void* q, const void* k, const void* v, const uint32_t* mask,
                             int64_t mask_b, int64_t mask_h, int64_t B, int64_t H, int64_t Nq,
                             int64_t Nk, int64_t d, int causal, float scale, int dtype,
                             int64_t n_sel, const int64_t* sel_bh, const int64_t* sel_row,
                             int64_t key_block, double* o64, double* lse64);
int fa_ref_bwd_head_masked_f64(const void* q, const void* k, const void* v, const void* dout,
                               const uint32_t* mask, int64_t mask_b, int64_t mask_h, int64_t B,
                               int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                               float scale, int dtype, int64_t bh, double* dq64, double* dk64,
                               double* dv64);

/* Whole-tensor host counterpart of the GPU backward: part 3 on every head, the
 * gradients rounded from fp64 to `dtype` (nearest-even) into dq, dk, dv. */
int fa_bwd_ref(const void* q, const void* k, const void* v, const void* dout, void* dq,
               void* dk, void* dv, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
               int causal, float scale, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* FA_ORACLE_H */
