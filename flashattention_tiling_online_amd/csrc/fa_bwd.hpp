// fa_bwd.hpp — gradients of the fused attention forward on gfx950 (bf16 / fp16 inputs).
//
// The backward pass recomputes the scores from Q, K and the forward's row log-sum-exp
// L instead of storing P (course page "05_flash_attention.py", flash_attention_backward;
// "Flash Attention" blog page, Algorithm 4):
//     P = exp(S - L),  dV = P^T dO,  dP = dO V^T,  D = rowsum(dO o O),
//     dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,
// with S = scale Q K^T masked as in the forward.  D uses the O the forward stored.
//
// Three kernels, no atomics, so the results are deterministic:
//   * fa_bwd_delta_kernel: D per query row (memory-bound, one row per D/4 threads);
//   * fa_bwd_dkv_kernel: one workgroup per 128-key tile (8 waves: 4 blocks of 32 keys,
//     lane = key, times the two 32-query halves of every 64-query tile), K and V
//     resident in LDS: S = Q K^T and dP = dO V^T, then dV^T += dO^T P and
//     dK^T += Q^T dS with P and dS rounded to T straight from the accumulators; the
//     two halves' partial sums meet in LDS at the end;
//   * fa_bwd_dq_kernel: one workgroup per 256-query tile for d = 128 (8 waves x 32
//     queries, lane = query, the forward's orientation; 128 queries for d = 64),
//     looping over 64-key tiles: S^T = K Q^T and dP^T = V dO^T with Q and dO in
//     registers, then dQ^T += K^T dS^T.
// Both main kernels stage the streamed tiles (Q and dO; K and V) as rows by DMA into
// two LDS buffers, a tile ahead, and read the operands that contract over the tile's
// rows (Q^T, dO^T; K^T) straight from those rows with the transposing LDS read
// (tr_operand, fa_tiles.hpp), so one barrier per tile covers the staging; exp is exp2
// with scale * log2(e) folded into one FMA and L taken in base 2.  With a caller mask (the blog page's Algorithm 4 recomputes P
// from mask(S)) a hidden (query, key) gets P = 0, which also covers the rows with no
// visible key (L = -inf, no gradient).
#pragma once

#include "fa_philox.hpp"
#include "fa_tiles.hpp"

namespace fa {

template <typename T>
struct BwdParams {
    const T* q;       // [bh, Nq, D]
    const T* k;       // [bh, Nk, D]
    const T* v;       // [bh, Nk, D]
    const T* o;       // [bh, Nq, D], the forward's output
    const T* dout;    // [bh, Nq, D]
    const float* lse; // [bh, Nq], the forward's natural-log row log-sum-exp
    float* delta;     // [bh, Nq], D = rowsum(dO o O) (written by the delta kernel)
    T* dq;            // [bh, Nq, D]
    T* dk;            // [bh, Nk, D]
    T* dv;            // [bh, Nk, D]
    int Nq, Nk;
    int n_tiles;      // tiles per head of the kernel's outer dimension
    float c2;         // scale * log2(e)
    float scale;
    DropParams drop;  // dropout on P (dropout instantiations only)
    // caller mask (masked instantiations only), as in FwdParams: rows of mask_w words,
    // head bh = b * H + h at mask + b * mask_sb + h * mask_sh
    const uint32_t* mask;
    int64_t mask_sb, mask_sh;
    int mask_w, H;
};

constexpr float kLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------------------
// D = rowsum(dO o O)
// ---------------------------------------------------------------------------

template <typename T, int D>
__global__ __launch_bounds__(256)
void fa_bwd_delta_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                         float* __restrict__ delta, int64_t rows)
{
    constexpr int TPR = D / 4;  // threads per row, 4 elements each
    typedef T T4 __attribute__((ext_vector_type(4)));
    const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
    const int t = (int)(threadIdx.x % TPR);
    float acc = 0.f;
    if (row < rows) {
        const T4 a = *reinterpret_cast<const T4*>(O + row * D + 4 * t);
        const T4 b = *reinterpret_cast<const T4*>(dO + row * D + 4 * t);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc += (float)a[e] * (float)b[e];
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m /= 2)
        acc += __shfl_xor(acc, m);
    if (row < rows && t == 0)
        delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 128 keys, lane = key
// ---------------------------------------------------------------------------

template <int D>
struct DkvTile {
    static constexpr int NW = 8;                 // waves: 4 key blocks x 2 query halves
    static constexpr int NT = 64 * NW;
    static constexpr int KEYS = 128;             // keys per workgroup
    static constexpr int TILE = 64;              // queries per step
    static constexpr int RSTR = 2 * D + 16;      // K and V rows (resident)
    // Q and dO rows: with 2D + 48 bytes the 16 rows of a ds_read_b128 pass fall in
    // distinct banks and the 4 rows of a half-wave's transposing read meet at most
    // 2-way (no stride makes both conflict-free)
    static constexpr int QSTR = 2 * D + 48;
    static constexpr int DC = D / 16;
    static constexpr int DB = D / 32;
    // LDS: K and V of the workgroup's keys (resident), then two staging buffers, each
    // the Q and dO rows of one 64-query tile, the 64 queries' L2 and D and the
    // caller-mask words [4 key words][64 queries]
    static constexpr int KS = 0;
    static constexpr int VS = KEYS * RSTR;
    static constexpr int STG0 = 2 * KEYS * RSTR;
    static constexpr int SDO = TILE * QSTR;
    static constexpr int SL = 2 * TILE * QSTR;
    static constexpr int SD = SL + TILE * 4;
    static constexpr int SM = SD + TILE * 4;
    static constexpr int STG = ((SM + 4 * TILE * 4 + 1023) / 1024) * 1024;
    static constexpr int LDS = STG0 + 2 * STG;
    static constexpr int QNB = TILE * QSTR / 1024;  // 1-KB DMA blocks per Q or dO tile
    static constexpr int QPW = (QNB + NW - 1) / NW;
    static_assert(TILE * QSTR % 1024 == 0 && STG0 % 1024 == 0, "tiles must be whole DMA blocks");
    // partial accumulators of the second query half, exchanged at the end
    static constexpr int XCH = 4 * 2 * DB * 16 * 64 * 4;
    static_assert(XCH <= LDS, "reduction buffer must fit the staging space");
    static constexpr int OSTR = 2 * 64 + 16;     // bytes per staged row of 64 dK or dV columns
    static_assert(4 * 2 * 32 * OSTR <= LDS, "the staged dK and dV rows must fit");
};

template <typename T, int D, bool CAUSAL, bool DROP = false, bool MASK = false>
__global__ __launch_bounds__(DkvTile<D>::NT) __attribute__((amdgpu_waves_per_eu(2)))
void fa_bwd_dkv_kernel(const BwdParams<T> prm)
{
    using P = DkvTile<D>;
    using M = Mfma16<T>;
    using vec = typename M::vec;
    typedef T T4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(1024))) char smem[P::LDS];
    const char* const sm = smem;
    const int Nq = prm.Nq, Nk = prm.Nk;

    const WorkItem wi = work_item((int)blockIdx.x, (int)gridDim.x, prm.n_tiles, CAUSAL);
    const int bh = wi.head;
    const int kt = wi.rank;  // key tile: heaviest (causal) first
    const int k0 = kt * P::KEYS;

    const int tid = (int)threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int kl = lane & 31;
    const int hh = lane >> 5;
    const int kblk = wave & 3;   // 32-key block of this wave
    const int qh = wave >> 2;    // query half of every 64-query tile
    const int kw0 = k0 + 32 * kblk;
    const int my_k = kw0 + kl;

    const T* Qh = prm.q + (size_t)bh * Nq * D;
    const T* dOh = prm.dout + (size_t)bh * Nq * D;
    const float* Lh = prm.lse + (size_t)bh * Nq;
    const float* Dh = prm.delta + (size_t)bh * Nq;
    const uint32_t* mslice = MASK ? mask_slice(prm, bh) : nullptr;

    // K and V rows of the workgroup's keys, resident for the whole loop (rows past Nk
    // read as zero; their gradients are not stored)
    {
        constexpr int CPR = (2 * D) / 16;
        const T* Kh = prm.k + (size_t)bh * Nk * D;
        const T* Vh = prm.v + (size_t)bh * Nk * D;
        const __amdgpu_buffer_rsrc_t rk = rows_rsrc<D>(Kh, k0, Nk);
        const __amdgpu_buffer_rsrc_t rv = rows_rsrc<D>(Vh, k0, Nk);
#pragma unroll
        for (int i = 0; i < (P::KEYS * CPR) / P::NT; ++i) {
            const int c = tid + i * P::NT;
            const int row = c / CPR, ch = c - (c / CPR) * CPR;
            const int src = (row * D + ch * 8) * 2, dst = row * P::RSTR + ch * 16;
            *reinterpret_cast<u32x4*>(smem + P::KS + dst) =
                __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, src, 0, 0));
            *reinterpret_cast<u32x4*>(smem + P::VS + dst) =
                __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, src, 0, 0));
        }
    }

    f32x16 dvt[P::DB], dkt[P::DB];
#pragma unroll
    for (int db = 0; db < P::DB; ++db) {
        dvt[db] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        dkt[db] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    }

    // query tiles: causal ones before the workgroup's first key see none of its keys
    const int nqt = (Nq + P::TILE - 1) / P::TILE;
    const int i0 = CAUSAL ? min(nqt, k0 / P::TILE) : 0;

    // staging of query tile i into buffer s, issued a tile ahead: the Q and dO rows by
    // DMA (rows past Nq read as zero), the 64 queries' L2 and D and the mask words
    // through registers, written to LDS at the end of the tile before
    int qsrc[P::QPW];
#pragma unroll
    for (int k = 0; k < P::QPW; ++k)
        qsrc[k] = dma_src<D>(wave + P::NW * k, lane, P::QSTR);
    auto stage_rows = [&](int i, int s) {
        char* const b = smem + P::STG0 + s * P::STG;
        stage_tile_asm<D, P::QNB, P::QPW, P::NW>(Qh, i, Nq, b, wave, qsrc);
        stage_tile_asm<D, P::QNB, P::QPW, P::NW>(dOh, i, Nq, b + P::SDO, wave, qsrc);
    };
    float n_l2 = 0.f, n_d = 0.f;
    uint32_t n_mw = 0u;
    auto load_small = [&](int i) {
        if (tid < P::TILE) {
            const int q = i * P::TILE + tid;
            // rows past Nq: P = exp2(-inf) = 0
            n_l2 = q < Nq ? Lh[q] * kLog2e : __builtin_inff();
            n_d = q < Nq ? Dh[q] : 0.f;
        }
        if (MASK && tid < 4 * P::TILE) {
            // word kw of query row q: the bits of keys k0 + 32 kw .. +31 (rows past Nq and
            // words past the row read as 0)
            const int q = i * P::TILE + (tid >> 2), kw = tid & 3;
            const int word = k0 / 32 + kw;
            n_mw = (q < Nq && word < prm.mask_w) ? mslice[(size_t)q * prm.mask_w + word] : 0u;
        }
    };
    auto store_small = [&](int s) {
        char* const b = smem + P::STG0 + s * P::STG;
        if (tid < P::TILE) {
            reinterpret_cast<float*>(b + P::SL)[tid] = n_l2;
            reinterpret_cast<float*>(b + P::SD)[tid] = n_d;
        }
        if (MASK && tid < 4 * P::TILE)
            reinterpret_cast<uint32_t*>(b + P::SM)[(tid & 3) * P::TILE + (tid >> 2)] = n_mw;
    };
    // all of this wave's memory operations complete (the DMA among them), then the
    // workgroup barrier
    auto barrier_all = [&]() {
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };

    const int rbase = kl * P::RSTR + hh * 16;   // K, V operand: row kl, chunk 8hh
    const int kbase = P::KS + 32 * kblk * P::RSTR + rbase;
    const int vbase = P::VS + 32 * kblk * P::RSTR + rbase;
    const int qbase = (32 * qh + kl) * P::QSTR + hh * 16;  // Q, dO row operand of this half
    // transposing reads of Q and dO (tr_operand): chunk 2qh + h of the tile
    const int tbase = (4 * hh + ((lane >> 2) & 3)) * P::QSTR + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    if (i0 < nqt) {
        stage_rows(i0, i0 & 1);
        load_small(i0);
        store_small(i0 & 1);
    }
    barrier_all();  // K, V and the first tile are staged
    for (int i = i0; i < nqt; ++i) {
        const int s = i & 1;
        if (i + 1 < nqt) {  // in flight while this tile is computed
            stage_rows(i + 1, s ^ 1);
            load_small(i + 1);
        }
        const char* const b = sm + P::STG0 + s * P::STG;
        const int qw = i * P::TILE + 32 * qh;  // first query of this wave's half
        // a half whose every query precedes every key of the block has nothing to add
        if (!(CAUSAL && qw + 31 < kw0)) {
            const bool diag = CAUSAL && (qw < kw0 + 31);
            // S = Q K^T and dP = dO V^T for the 32 queries of this half
            f32x16 sacc = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
            f32x16 dp = sacc;
#pragma unroll
            for (int c = 0; c < P::DC; ++c) {
                const vec kf = *reinterpret_cast<const vec*>(sm + kbase + 32 * c);
                const vec a = *reinterpret_cast<const vec*>(b + qbase + 32 * c);
                sacc = M::mma(a, kf, sacc);
                const vec vf = *reinterpret_cast<const vec*>(sm + vbase + 32 * c);
                const vec a2 = *reinterpret_cast<const vec*>(b + P::SDO + qbase + 32 * c);
                dp = M::mma(a2, vf, dp);
            }
            // P = 2^(s c2 - L2), dS = P (dP - D); register r holds query
            // qw + 8(r/4) + 4hh + r%4.  With dropout Z: dV takes P o Z, dS takes dP o Z.
            vec pp[2], ps[2];
            uint32_t dw[4];  // group g: queries i TILE + 32qh + 8g + 4hh + 0..3
            if (DROP)
                drop_words_k4(prm.drop, bh, i * P::TILE + 32 * qh + 4 * hh, my_k, dw);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int qo = 32 * qh + 8 * g + 4 * hh;
                const f32x4 l2 = *reinterpret_cast<const f32x4*>(b + P::SL + qo * 4);
                const f32x4 dd = *reinterpret_cast<const f32x4*>(b + P::SD + qo * 4);
                u32x4 mw = {0u, 0u, 0u, 0u};
                if (MASK)
                    mw = *reinterpret_cast<const u32x4*>(b + P::SM + (kblk * P::TILE + qo) * 4);
                uint32_t bytes = 0;
                if (DROP)
                    bytes = dw[g];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    float p = exp2_fast(fmaf(sacc[r], prm.c2, -l2[e]));
                    if (diag && my_k > i * P::TILE + qo + e)
                        p = 0.f;  // key after the query
                    if (MASK && !((mw[e] >> kl) & 1u))
                        p = 0.f;  // key hidden by the caller's mask (also for a row with L = -inf)
                    if (DROP) {
                        const float z = drop_keep(bytes, e, prm.drop.t) ? prm.drop.keep_scale : 0.f;
                        pp[r >> 3][r & 7] = (T)(p * z);
                        ps[r >> 3][r & 7] = (T)(p * (dp[r] * z - dd[e]));
                    } else {
                        pp[r >> 3][r & 7] = (T)p;
                        ps[r >> 3][r & 7] = (T)(p * (dp[r] - dd[e]));
                    }
                }
            }
            // dV^T += dO^T P, dK^T += Q^T dS over chunks 2qh, 2qh+1 of the tile, the
            // transposed operands read straight from the row tiles
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int cc = 2 * qh + h;
#pragma unroll
                for (int db = 0; db < P::DB; ++db) {
                    const char* const tp = b + tbase + 16 * cc * P::QSTR + 64 * db;
                    dvt[db] = M::mma(tr_operand<P::QSTR, vec>(tp + P::SDO), pp[h], dvt[db]);
                    dkt[db] = M::mma(tr_operand<P::QSTR, vec>(tp), ps[h], dkt[db]);
                }
            }
        }
        if (i + 1 < nqt)
            store_small(s ^ 1);
        barrier_all();  // the next tile has landed; this one is consumed
    }

    // the second query half hands its partial sums to the first through LDS
    wg_barrier();
    float* xch = reinterpret_cast<float*>(smem);
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                xch[(((kblk * 2 + 0) * P::DB + db) * 16 + r) * 64 + lane] = dkt[db][r];
                xch[(((kblk * 2 + 1) * P::DB + db) * 16 + r) * 64 + lane] = dvt[db][r];
            }
    }
    wg_barrier();
    if (qh == 0) {
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dkt[db][r] += xch[(((kblk * 2 + 0) * P::DB + db) * 16 + r) * 64 + lane];
                dvt[db][r] += xch[(((kblk * 2 + 1) * P::DB + db) * 16 + r) * 64 + lane];
            }
    }
    wg_barrier();  // the exchange is read: its space takes the rows of dK and dV
    if (qh == 1)
        return;
    // epilogue: accumulator register r of block db holds d = 32db + 8(r/4) + 4hh + r%4.
    // The rows go through this wave's LDS rows, 64 columns at a time, so that each
    // store writes 128 bytes of 8 rows rather than 8 bytes of 32 rows.
    char* const kst = smem + kblk * 2 * 32 * P::OSTR;
    char* const vst = kst + 32 * P::OSTR;
    T* const dkh = prm.dk + (size_t)bh * Nk * D;
    T* const dvh = prm.dv + (size_t)bh * Nk * D;
#pragma unroll
    for (int half = 0; half < D / 64; ++half) {
#pragma unroll
        for (int db = 2 * half; db < 2 * half + 2; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                T4 wk, wv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wk[e] = (T)(dkt[db][4 * a + e] * prm.scale);
                    wv[e] = (T)dvt[db][4 * a + e];
                }
                const int off = kl * P::OSTR + 2 * (32 * (db - 2 * half) + 8 * a + 4 * hh);
                *reinterpret_cast<T4*>(kst + off) = wk;
                *reinterpret_cast<T4*>(vst + off) = wv;
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 8 * i + (lane >> 3);
            const int ch = lane & 7;
            const u32x4 pk = *reinterpret_cast<const u32x4*>(kst + r * P::OSTR + 16 * ch);
            const u32x4 pv = *reinterpret_cast<const u32x4*>(vst + r * P::OSTR + 16 * ch);
            if (kw0 + r < Nk) {
                *reinterpret_cast<u32x4*>(dkh + (size_t)(kw0 + r) * D + 64 * half + 8 * ch) = pk;
                *reinterpret_cast<u32x4*>(dvh + (size_t)(kw0 + r) * D + 64 * half + 8 * ch) = pv;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 128 queries, lane = query
// ---------------------------------------------------------------------------

template <int D>
struct DqTile {
    // d = 128: 8 waves (256 queries) per workgroup, one per CU; d = 64: 4 waves (128
    // queries), two per CU
    static constexpr int NW = D == 128 ? 8 : 4;
    static constexpr int NT = 64 * NW;
    static constexpr int ROWS = 32 * NW;        // queries per workgroup
    static constexpr int TILE = 64;             // keys per step
    static constexpr int RSTR = 2 * D + 16;     // V rows
    // K rows: read as rows (S^T = K Q^T) and transposed (dQ^T += K^T dS^T); with 2D + 48
    // bytes the first is conflict-free and the second meets at most 2-way
    static constexpr int KSTR = 2 * D + 48;
    static constexpr int DC = D / 16;
    static constexpr int DB = D / 32;
    // LDS: two buffers each of K rows and V rows, DMA'd a tile ahead
    static constexpr int KB = TILE * KSTR;
    static constexpr int VB = TILE * RSTR;
    static constexpr int VOFF = 2 * KB;
    static constexpr int LDS = 2 * KB + 2 * VB;
    static constexpr int KNB = KB / 1024;       // 1-KB DMA blocks per K or V tile
    static constexpr int VNB = VB / 1024;
    static constexpr int KPW = (KNB + NW - 1) / NW;
    static constexpr int VPW = (VNB + NW - 1) / NW;
    static_assert(KB % 1024 == 0 && VB % 1024 == 0, "tiles must be whole DMA blocks");
    static constexpr int OSTR = 2 * 64 + 16;     // bytes per staged row of 64 dQ columns
    static_assert(NW * 32 * OSTR <= LDS, "the staged dQ rows must fit the tiles");
};

template <typename T, int D, bool CAUSAL, bool DROP = false, bool MASK = false>
__global__ __launch_bounds__(DqTile<D>::NT) __attribute__((amdgpu_waves_per_eu(2)))
void fa_bwd_dq_kernel(const BwdParams<T> prm)
{
    using P = DqTile<D>;
    using M = Mfma16<T>;
    using vec = typename M::vec;
    typedef T T4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(1024))) char smem[P::LDS];
    const char* const sm = smem;
    const int Nq = prm.Nq, Nk = prm.Nk;

    const WorkItem wi = work_item((int)blockIdx.x, (int)gridDim.x, prm.n_tiles, CAUSAL);
    const int bh = wi.head;
    const int qt = CAUSAL ? prm.n_tiles - 1 - wi.rank : wi.rank;  // longest rows first
    const int q0 = qt * P::ROWS;

    const int tid = (int)threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int ql = lane & 31;
    const int hh = lane >> 5;
    const int qw0 = q0 + 32 * wave;
    const int my_q = qw0 + ql;

    const T* Kh = prm.k + (size_t)bh * Nk * D;
    const T* Vh = prm.v + (size_t)bh * Nk * D;

    // key tiles, as in the forward: causal tiles after the workgroup's last query are
    // skipped, a wave stops after its own last query, only its last tile is masked
    int nkt = (Nk + P::TILE - 1) / P::TILE;
    if (CAUSAL)
        nkt = min(nkt, (min(q0 + P::ROWS, Nq) - 1) / P::TILE + 1);
    const bool wave_active = qw0 < Nq;
    int n_w = wave_active ? nkt : 0;
    if (CAUSAL && wave_active)
        n_w = min(nkt, min(qw0 + 31, Nq - 1) / P::TILE + 1);

    // staging: K and V rows of key tile j by DMA into buffer j % 2, issued a tile ahead
    int ksrc[P::KPW], vsrc[P::VPW];
#pragma unroll
    for (int i = 0; i < P::KPW; ++i)
        ksrc[i] = dma_src<D>(wave + P::NW * i, lane, P::KSTR);
#pragma unroll
    for (int i = 0; i < P::VPW; ++i)
        vsrc[i] = dma_src<D>(wave + P::NW * i, lane, P::RSTR);
    auto stage = [&](int j, int buf) {
        stage_tile_asm<D, P::KNB, P::KPW, P::NW>(Kh, j, Nk, smem + buf * P::KB, wave, ksrc);
        stage_tile_asm<D, P::VNB, P::VPW, P::NW>(Vh, j, Nk, smem + P::VOFF + buf * P::VB, wave, vsrc);
    };
    // all of this wave's memory operations complete (the DMA among them), then the
    // workgroup barrier
    auto barrier_all = [&]() {
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };
    if (0 < nkt)
        stage(0, 0);

    // Q and dO rows of this lane's query as the B operands
    vec qf[P::DC], df[P::DC];
#pragma unroll
    for (int c = 0; c < P::DC; ++c) {
        u32x4 rq = {0u, 0u, 0u, 0u}, rd = {0u, 0u, 0u, 0u};
        if (my_q < Nq) {
            const size_t off = ((size_t)bh * Nq + my_q) * D + 16 * c + 8 * hh;
            rq = *reinterpret_cast<const u32x4*>(prm.q + off);
            rd = *reinterpret_cast<const u32x4*>(prm.dout + off);
        }
        qf[c] = __builtin_bit_cast(vec, rq);
        df[c] = __builtin_bit_cast(vec, rd);
    }
    const float l2 = my_q < Nq ? prm.lse[(size_t)bh * Nq + my_q] * kLog2e : 0.f;
    const float dd = my_q < Nq ? prm.delta[(size_t)bh * Nq + my_q] : 0.f;

    // caller mask: this lane's row, the two words of a key tile loaded a tile ahead
    // (words past the row and rows past Nq read as 0 through the resource's bound)
    const __amdgpu_buffer_rsrc_t mrs = mask_rsrc(MASK ? mask_slice(prm, bh) : nullptr, q0, P::ROWS,
                                                 Nq, MASK ? prm.mask_w : 0);
    const int mrow_off = MASK ? (my_q - q0) * prm.mask_w * 4 : 0;
    uint32_t mw[2] = {0u, 0u};
    auto load_mask = [&](int t) {
        mw[0] = __builtin_amdgcn_raw_buffer_load_b32(mrs, mrow_off + 8 * t, 0, 0);
        mw[1] = __builtin_amdgcn_raw_buffer_load_b32(mrs, mrow_off + 8 * t + 4, 0, 0);
    };
    if (MASK && 0 < n_w)
        load_mask(0);

    f32x16 dqt[P::DB];
#pragma unroll
    for (int db = 0; db < P::DB; ++db)
        dqt[db] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    const int kbase = ql * P::KSTR + hh * 16;   // K row operand: row ql, chunk 8hh
    const int vbase = ql * P::RSTR + hh * 16;
    // transposing reads of K (tr_operand): chunk cc of the tile, 32 dims per block
    const int tbase = (4 * hh + ((lane >> 2) & 3)) * P::KSTR + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    barrier_all();  // K_0 and V_0 have landed
    for (int j = 0; j < nkt; ++j) {
        const int buf = j & 1;
        if (j + 1 < nkt)  // in flight while this tile is computed
            stage(j + 1, buf ^ 1);
        if (j < n_w) {
            const char* const kt = sm + buf * P::KB;
            const char* const vr = sm + P::VOFF + buf * P::VB;
            // S^T = K Q^T, dP^T = V dO^T: register r of block kb holds key
            // 32kb + 8(r/4) + 4hh + r%4 of the tile
            f32x16 st[2], dpt[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                st[kb] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
                dpt[kb] = st[kb];
#pragma unroll
                for (int c = 0; c < P::DC; ++c) {
                    const vec a = *reinterpret_cast<const vec*>(kt + kbase + 32 * kb * P::KSTR + 32 * c);
                    st[kb] = M::mma(a, qf[c], st[kb]);
                    const vec b = *reinterpret_cast<const vec*>(vr + vbase + 32 * kb * P::RSTR + 32 * c);
                    dpt[kb] = M::mma(b, df[c], dpt[kb]);
                }
            }
            const int key0 = j * P::TILE;
            const bool mask = (key0 + P::TILE > Nk) || (CAUSAL && key0 + P::TILE - 1 > qw0);
            const int last = CAUSAL ? min(Nk - 1, my_q) : Nk - 1;
            // this lane's caller-mask bits of the tile, shifted so that register r of block
            // kb finds its key at bit 8 (r / 4) + r % 4 of cm[kb]; then the next tile's words
            uint32_t cm[2] = {~0u, ~0u};
            if (MASK) {
                cm[0] = mw[0] >> (4 * hh);
                cm[1] = mw[1] >> (4 * hh);
                if (j + 1 < n_w)
                    load_mask(j + 1);
            }
            vec ps[4];
            uint32_t dw[8];  // group 2cc + g: keys key0 + 16cc + 8g + 4hh + 0..3
            if (DROP)
                drop_words_q8(prm.drop, bh, my_q, key0 + 4 * hh, dw);
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                // chunk cc holds keys 16cc + 4hh + 0..3 (e < 4) and 16cc + 8 + 4hh + 0..3
                uint32_t bytes[2] = {0u, 0u};
                if (DROP) {
                    bytes[0] = dw[2 * cc];
                    bytes[1] = dw[2 * cc + 1];
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kb = cc >> 1, r = 8 * (cc & 1) + e;
                    float p = exp2_fast(fmaf(st[kb][r], prm.c2, -l2));
                    if (mask && key0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3) > last)
                        p = 0.f;
                    if (MASK && !((cm[kb] >> (8 * (r >> 2) + (r & 3))) & 1u))
                        p = 0.f;  // key hidden by the caller's mask (also for a row with L = -inf)
                    float dpz = dpt[kb][r];
                    if (DROP)
                        dpz *= drop_keep(bytes[e >> 2], e & 3, prm.drop.t) ? prm.drop.keep_scale : 0.f;
                    ps[cc][e] = (T)(p * (dpz - dd));
                }
            }
            // dQ^T += K^T dS^T, K^T read transposed from the K rows
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                for (int db = 0; db < P::DB; ++db)
                    dqt[db] = M::mma(tr_operand<P::KSTR, vec>(kt + tbase + 16 * cc * P::KSTR + 64 * db),
                                     ps[cc], dqt[db]);
        }
        barrier_all();  // the next tile has landed; this one is consumed
    }

    // dQ rows through this wave's LDS rows, 64 columns at a time (the K and V tiles
    // are consumed after the barrier), so that each store writes 128 bytes of 8 rows
    wg_barrier();
    char* const ost = smem + wave * 32 * P::OSTR;
    T* const dqh = prm.dq + (size_t)bh * Nq * D;
#pragma unroll
    for (int half = 0; half < D / 64; ++half) {
#pragma unroll
        for (int db = 2 * half; db < 2 * half + 2; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                T4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = (T)(dqt[db][4 * a + e] * prm.scale);
                *reinterpret_cast<T4*>(ost + ql * P::OSTR + 2 * (32 * (db - 2 * half) + 8 * a + 4 * hh)) = w;
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 8 * i + (lane >> 3);
            const int ch = lane & 7;
            const u32x4 piece = *reinterpret_cast<const u32x4*>(ost + r * P::OSTR + 16 * ch);
            if (qw0 + r < Nq)
                *reinterpret_cast<u32x4*>(dqh + (size_t)(qw0 + r) * D + 64 * half + 8 * ch) = piece;
        }
    }
}

}  // namespace fa
