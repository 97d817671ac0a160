/*
 * fa.h — C-ABI of the MI355X (gfx950) fused attention forward library, libfa.so.
 *
 * The forward entry points compute, for every batch b and head h,
 *
 *     S = scale * Q[b,h] K[b,h]^T            (Nq x Nk, never written to memory)
 *     S[q,k] = -inf where causal and k > q   (key k visible to query q iff k <= q)
 *     O[b,h] = softmax_rows(S) V[b,h]
 *     L[b,h,q] = ln sum_k exp(S[q,k])        (the row logsumexp, natural log)
 *
 * tiled over query row-blocks and key/value column-blocks with the online-softmax
 * (m, l, O~) recurrence, so that the score matrix stays on chip.  Definitions:
 *   - the operation and the returned L = m + log l: the "05_flash_attention.py"
 *     course page (semidirectx.com, CS336 lecture 5), standard_attention and
 *     flash_attention_forward;
 *   - the scale tau applied to Q K^T and the mask: the "Flash Attention" blog page
 *     (blog.cyberangel.work), Algorithm 2;
 *   - the causal rule (k visible to q iff k <= q, top-left aligned): the course
 *     page's triu(1) mask and its causal block skip.
 *
 * The library allocates nothing, keeps no state between calls and never prints.
 * Every call is re-entrant.  Link with -lfa (it depends on the HIP runtime only).
 */
#ifndef FA_H
#define FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Under C++ the two enums below have int as their fixed underlying type, so any int a
 * C caller passes is a value of the type there too; the entry points refuse the ones
 * they do not know (FA_ERR_INVALID_ARG). */
#ifdef __cplusplus
#define FA_ENUM_INT : int
#else
#define FA_ENUM_INT
#endif

/* Element type of q, k, v and o.  lse is always fp32. */
typedef enum FA_ENUM_INT {
    FA_DTYPE_F32 = 0,  /* IEEE binary32 */
    FA_DTYPE_F16 = 1,  /* IEEE binary16 */
    FA_DTYPE_BF16 = 2  /* bfloat16 (upper half of binary32) */
} fa_dtype_t;

typedef enum FA_ENUM_INT {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, Nk = 0 with queries,
                               non-positive or non-finite scale, unknown dtype, size limit */
    FA_ERR_UNSUPPORTED = 2, /* head size d outside {64, 128} */
    FA_ERR_LAUNCH = 3,      /* the HIP runtime rejected the kernel launch */
    FA_ERR_SCRATCH = 4      /* fa_fwd_split_static: the problem needs more scratch than
                               FA_STATIC_SCRATCH_BYTES */
} fa_status_t;

/* hipStream_t without the HIP headers: pass the stream handle (0 = default stream). */
typedef void* fa_stream_t;

/*
 * fa_fwd — fused attention forward on the GPU.
 *
 * Arguments (all pointers are DEVICE pointers owned by the caller):
 *   q    [B, H, Nq, d]  element type `dtype`, contiguous, d fastest
 *   k    [B, H, Nk, d]  same
 *   v    [B, H, Nk, d]  same
 *   o    [B, H, Nq, d]  output, element type `dtype`; rounded from fp32 to nearest-even
 *   lse  [B, H, Nq]     output, fp32, natural-log row logsumexp of the scaled, masked scores
 *   B, H, Nq, Nk        batch, heads, query and key/value lengths (any values >= 0 that
 *                       fit the limits below; not restricted to tile multiples)
 *   d                   head size: 64 or 128
 *   causal              0: every key visible; 1: key k visible to query q iff k <= q
 *                       (0-based, top-left aligned also when Nq != Nk)
 *   scale               multiplies Q K^T before the softmax (usually 1/sqrt(d));
 *                       must be finite and > 0
 *   dtype               element type of q, k, v and o
 *   stream              HIP stream the kernel is enqueued on
 *
 * Alignment: q, k, v and o must be 16-byte aligned, lse 4-byte aligned.  The output
 * buffers must not overlap the inputs.
 *
 * Behaviour:
 *   - returns before the kernel completes (asynchronous on `stream`);
 *   - B*H*Nq == 0: nothing to compute, returns FA_OK without touching the GPU or
 *     any buffer (the pointers may then be NULL; dtype, d, causal and scale are still
 *     validated);
 *   - Nk == 0 with queries present: FA_ERR_INVALID_ARG (softmax over no keys);
 *   - every argument error is reported before any HIP call;
 *   - NaN or Inf in the inputs propagate to the affected rows;
 *   - limits: Nq*d and Nk*d below 2^31 (per-head offsets are 32-bit), B*H below 2^31,
 *     and ceil(Nq / fa_tile_rows(...)) * B * H below 2^31 (the 1-D grid); otherwise
 *     FA_ERR_INVALID_ARG.
 * Results are deterministic: the same inputs give bitwise-identical outputs.
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                   float scale, fa_dtype_t dtype, fa_stream_t stream);

/*
 * fa_fwd_masked — fa_fwd with a caller's boolean mask on the scores: the "Flash
 * Attention" blog page (blog.cyberangel.work), Algorithm 2, S_masked = mask(S) before
 * the softmax.  A hidden (q, k) gets S[q, k] = -inf, on top of the causal rule when
 * causal = 1 (a key must be allowed by both).
 *
 *   mask        DEVICE buffer of uint32 words [mask_b, mask_h, Nq, W], W = ceil(Nk / 32),
 *               4-byte aligned, owned by the caller: row (b, h, q) holds key k in bit
 *               k % 32 of word k / 32, set = visible (bits for keys >= Nk are ignored)
 *   mask_b      1 (one mask for every batch) or B
 *   mask_h      1 (one mask for every head) or H
 *   other arguments as fa_fwd.
 *
 * A query row with no visible key has no softmax; it gets O = 0 and L = -inf (the
 * identity of the (+) merge of partial states, as fa_fwd_split's empty ranges).
 * Behaviour, limits and errors as fa_fwd (FA_ERR_INVALID_ARG also for a null or
 * misaligned mask or mask_b / mask_h outside {1, B} / {1, H}); every dtype and d of
 * fa_fwd.  Deterministic.
 */
fa_status_t fa_fwd_masked(const void* q, const void* k, const void* v, const uint32_t* mask,
                          int64_t mask_b, int64_t mask_h, void* o, float* lse, int64_t B,
                          int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                          fa_dtype_t dtype, fa_stream_t stream);

/*
 * fa_fwd_split — the same result as fa_fwd, computed over key ranges in parallel and
 * merged; for grids that fa_fwd leaves under-filled (few heads, short query
 * sequences, long key sequences).
 *
 * The keys are cut into ranges of whole 64-key tiles: with nkt = ceil(Nk / 64) tiles,
 * s = min(n_splits, nkt) and t = ceil(nkt / s) tiles per range, range r covers keys
 * [64*t*r, min(64*t*(r+1), Nk)) and there are ceil(nkt / t) <= n_splits ranges.  Each
 * range leaves, per query row, a partial state in fp32: the normalised partial output
 * O_r and its log-sum-exp L_r (L_r = -inf and O_r = 0 where the range holds no key
 * visible to the row).  A second kernel folds them with the (+) operator of the
 * "Flash Attention" blog page (blog.cyberangel.work, the online-softmax merge of
 * (m, d, o~) states, associative and commutative) in log-sum-exp form:
 *     L = log sum_r exp(L_r),   O = sum_r exp(L_r - L) O_r,
 * then rounds O to `dtype` (nearest-even).  The result equals fa_fwd's up to fp32
 * rounding order.
 *
 * Arguments as fa_fwd, plus:
 *   n_splits         requested number of key ranges, 1 .. 256 (fewer are used when
 *                    Nk has fewer 64-key tiles); when only one range results, the
 *                    unsplit kernel runs and the workspace is not touched
 *   workspace        DEVICE buffer owned by the caller, 16-byte aligned, at least
 *                    fa_fwd_split_workspace(B, H, Nq, d, n_splits) bytes; it holds the
 *                    partials: O_r as fp32 [n_splits, B, H, Nq, d] at offset 0, then
 *                    L_r as fp32 [n_splits, B, H, Nq] at the next multiple of 256 bytes
 *                    (ranges beyond the number used are not written)
 *   workspace_bytes  its size in bytes
 *
 * Behaviour: as fa_fwd (validation first, asynchronous, deterministic), and
 * FA_ERR_INVALID_ARG for n_splits outside 1 .. 256 or a missing, misaligned or too
 * small workspace when more than one range is used.  Two kernels are enqueued in
 * order on `stream`; the workspace must not be reused until they complete.
 */
fa_status_t fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                         float scale, fa_dtype_t dtype, int n_splits, void* workspace,
                         int64_t workspace_bytes, fa_stream_t stream);

/* Workspace bytes fa_fwd_split needs for (B, H, Nq, d, n_splits); -1 for arguments
 * it would reject (negative sizes, d outside {64, 128}, n_splits outside 1 .. 256) and
 * for sizes whose byte count does not fit in int64. */
int64_t fa_fwd_split_workspace(int64_t B, int64_t H, int64_t Nq, int64_t d, int n_splits);

/* Size of the library's static scratch buffer (fa_fwd_split_static), per GPU. */
#define FA_STATIC_SCRATCH_BYTES (64LL << 20)

/*
 * fa_fwd_split_static — fa_fwd_split without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code being captured
 * into a HIP graph, tight serving loops, harnesses that forbid hipMalloc.  The partial
 * states live in a static device array of FA_STATIC_SCRATCH_BYTES (64 MiB) that the
 * library holds on every GPU it runs on until the process ends; its address on a GPU
 * is looked up once, on the first call with that GPU current.
 *
 * Arguments, result and behaviour as fa_fwd_split (same kernels, same bits), with the
 * workspace replaced by that array.  The problem must fit it:
 * fa_fwd_split_workspace(B, H, Nq, d, n_splits) <= FA_STATIC_SCRATCH_BYTES when more
 * than one key range results, else FA_ERR_SCRATCH (before any HIP call).  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (on concurrent
 * streams, or before the previous call's kernels have finished on another stream)
 * race and give wrong results; calls in order on one stream are safe.  The array
 * keeps the last call's partials; nothing in it needs to start at zero (every partial
 * the merge reads is written first by the same call).  FA_ERR_LAUNCH if the array's
 * address cannot be obtained on the current GPU.
 */
fa_status_t fa_fwd_split_static(const void* q, const void* k, const void* v, void* o, float* lse,
                                int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                int causal, float scale, fa_dtype_t dtype, int n_splits,
                                fa_stream_t stream);

/*
 * fa_merge — fold partial attention states over disjoint key ranges into the final
 * output (the second half of fa_fwd_split, for partials computed elsewhere, e.g. one
 * part per GPU of a key-sharded sequence).  Definition: as in fa_fwd_split above.
 *
 *   o_parts    [n_parts, B, H, Nq, d] fp32 DEVICE buffer: O_r, the normalised partial
 *              output of key range r (16-byte aligned)
 *   lse_parts  [n_parts, B, H, Nq] fp32: L_r, natural-log log-sum-exp of range r's
 *              scaled, masked scores; -inf marks a range with no visible key (its O_r
 *              is then ignored)
 *   o          [B, H, Nq, d] output in `dtype`, rounded to nearest-even (16-byte aligned)
 *   lse        [B, H, Nq] fp32 output, log sum_r exp(L_r)
 * A row whose every L_r is -inf gets O = 0 and L = -inf.  n_parts >= 1; d 64 or 128
 * (else FA_ERR_UNSUPPORTED); B*H*Nq == 0 returns FA_OK without touching anything.
 * Asynchronous on `stream`; errors are reported before any HIP call.
 */
fa_status_t fa_merge(const float* o_parts, const float* lse_parts, int n_parts, int64_t B,
                     int64_t H, int64_t Nq, int64_t d, void* o, float* lse, fa_dtype_t dtype,
                     fa_stream_t stream);

/* A key-range count for fa_fwd_split that fills the GPU (256 CUs) when fa_fwd's grid of
 * B*H*ceil(Nq / fa_tile_rows(...)) workgroups would not: 1 when that grid already
 * fills it, otherwise enough ranges to, keeping at least eight 64-key tiles per range
 * (two for fp32) and at most 16 ranges.  0 for unsupported or empty arguments. */
int fa_split_hint(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                  fa_dtype_t dtype);

/*
 * fa_bwd — gradients of the forward above by recomputation: from Q, K, V, the
 * forward's O and L and the output gradient dO, the gradients of sum(dO o O):
 *
 *     P = exp(S - L)              (S scaled and masked as in fa_fwd)
 *     dV = P^T dO,  dP = dO V^T,  D = rowsum(dO o O),  dS = P o (dP - D),
 *     dQ = scale dS K,  dK = scale dS^T Q
 *
 * as the "05_flash_attention.py" course page (flash_attention_backward) and the
 * "Flash Attention" blog page (Algorithm 4 and the softmax-Jacobian derivation: D_i =
 * P_i . dP_i = do_i . o_i) define them.  P is never stored; D uses the O passed in.
 *
 * Arguments (DEVICE pointers owned by the caller, contiguous, d fastest):
 *   q, o, dout  [B, H, Nq, d]  `dtype`; o and lse as fa_fwd returned them
 *   k, v        [B, H, Nk, d]  `dtype`
 *   lse         [B, H, Nq]     fp32
 *   dq          [B, H, Nq, d]  output, `dtype`, rounded to nearest-even
 *   dk, dv      [B, H, Nk, d]  outputs, same
 *   B, H, Nq, Nk, d, causal, scale: as fa_fwd
 *   dtype       FA_DTYPE_BF16 or FA_DTYPE_F16 (FA_DTYPE_F32: FA_ERR_UNSUPPORTED)
 *   workspace   DEVICE buffer, 16-byte aligned, at least fa_bwd_workspace(B, H, Nq, d)
 *               bytes: D as fp32 [B, H, Nq]
 *
 * Alignment: as fa_fwd (16 bytes for every tensor, 4 for lse).  Behaviour:
 * asynchronous on `stream` (three kernels, in order); deterministic (no atomics:
 * bitwise-identical results for the same inputs); every argument error before any
 * HIP call.  B*H == 0, or Nq == Nk == 0: FA_OK, nothing touched.  Nq == 0 < Nk:
 * dk = dv = 0 are written (q, o, lse, dout, dq and the workspace may be NULL).
 * Nk == 0 < Nq: FA_ERR_INVALID_ARG.  Limits as fa_fwd, with 128-row tiles.
 */
fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                   int64_t Nq, int64_t Nk, int64_t d, int causal, float scale, fa_dtype_t dtype,
                   void* workspace, int64_t workspace_bytes, fa_stream_t stream);

/* Workspace bytes fa_bwd needs (D as fp32, rounded up to 256); -1 for negative sizes,
 * d outside {64, 128}, or sizes whose byte count does not fit in int64. */
int64_t fa_bwd_workspace(int64_t B, int64_t H, int64_t Nq, int64_t d);

/*
 * fa_bwd_masked — fa_bwd for the forward of fa_fwd_masked: the "Flash Attention" blog
 * page's Algorithm 4 recomputes P from mask(S), so a hidden (q, k) has P = 0 and adds
 * nothing to dQ, dK or dV; a query row with no visible key (L = -inf) has no gradient
 * (dQ row 0).  mask, mask_b, mask_h: as fa_fwd_masked (the same array the forward
 * used; with Nq == 0 it is not read and may be NULL).  Other arguments, behaviour and
 * errors as fa_bwd; dtype BF16 or F16.
 */
fa_status_t fa_bwd_masked(const void* q, const void* k, const void* v, const uint32_t* mask,
                          int64_t mask_b, int64_t mask_h, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                          int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                          fa_dtype_t dtype, void* workspace, int64_t workspace_bytes,
                          fa_stream_t stream);

/*
 * fa_fwd_dropout / fa_bwd_dropout — the forward and backward above with dropout on P.
 * The "Flash Attention" blog page (Algorithm 2) drops entries of P after the softmax
 * and multiplies the kept ones by 1/(1 - p): O = (P o Z) V with L unchanged (the
 * logsumexp of the undropped scores); its Algorithm 4 regenerates the same Z from the
 * saved generator state and uses P_dropped = P o Z for dV and dP o Z in dS:
 *
 *     dV = (P o Z)^T dO,  dS = P o (dP o Z - D),  D = rowsum(dO o O)
 *
 * The pages name no generator.  Z here: Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC'11) with key (seed bits 0-31,
 * seed bits 32-63) and counter (k / 4, q / 4, b * H + h, 0); element (q, k) of head
 * b * H + h takes byte 4 (q % 4) + k % 4 of the output (word q % 4, bits 8 (k % 4) ..
 * 8 (k % 4) + 7) and is dropped iff that byte is below t = round(256 p_drop); a kept
 * element is multiplied by 256 / (256 - t).  The drop probability is thus t / 256,
 * p_drop rounded to a multiple of 1/256.  The same (seed, p_drop) in both calls gives
 * the same Z, independent of tile shapes and launch order.
 *
 * Arguments as fa_fwd / fa_bwd, plus:
 *   p_drop  drop probability, 0 <= p_drop < 1 with round(256 p_drop) <= 255, else
 *           FA_ERR_INVALID_ARG; p_drop that rounds to t = 0 gives fa_fwd's / fa_bwd's
 *           result
 *   seed    the generator key (any value)
 * dtype must be FA_DTYPE_BF16 or FA_DTYPE_F16 (FA_DTYPE_F32: FA_ERR_UNSUPPORTED).
 * Behaviour, ownership, limits and the workspace of fa_bwd_dropout: as fa_fwd / fa_bwd.
 */
fa_status_t fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                           float scale, float p_drop, uint64_t seed, fa_dtype_t dtype,
                           fa_stream_t stream);
fa_status_t fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                           float scale, float p_drop, uint64_t seed, fa_dtype_t dtype,
                           void* workspace, int64_t workspace_bytes, fa_stream_t stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* fa_status_str(fa_status_t status);

/* Query-tile height (rows per workgroup) the library uses for (dtype, d, causal);
 * 0 if the combination is unsupported.  Lets a caller size sample checks and
 * compute the grid the library launches: ceil(Nq / rows) * B * H workgroups. */
int fa_tile_rows(fa_dtype_t dtype, int64_t d, int causal);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
