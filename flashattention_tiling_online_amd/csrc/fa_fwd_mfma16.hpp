// fa_fwd_mfma16.hpp — fused attention forward for bf16 / fp16 inputs on gfx950.
//
// The algorithm is the query-outer, key-inner online-softmax recurrence of the
// course page "05_flash_attention.py" (flash_attention_forward): per query tile
// m = -inf, l = 0, O~ = 0; for each key/value tile, left to right:
//     S = Q_i K_j^T * scale,  m_new = max(m, rowmax S),  P = exp(S - m_new),
//     alpha = exp(m - m_new), l = alpha l + rowsum P, O~ = alpha O~ + P V_j;
// at the end O = O~ / l and L = m + log l.  The unnormalised O~ is rescaled by
// exp(m_old - m_new) alone, as in the "Flash Attention" blog page's (+) operator
// on (m, d, o~).  Key tiles wholly in the causal future are skipped and only
// tiles that straddle the diagonal (or the ragged end of the keys) are masked
// (course page, causal branch of flash_attention_forward).
//
// gfx950 mapping (designed for CDNA4, not taken from the pages' NVIDIA design):
//   * workgroup = 4 wave64s = 128 query rows; wave w owns rows [32w, 32w+32);
//     2 workgroups per CU, so each SIMD interleaves two waves;
//   * both contractions on v_mfma_f32_32x32x16_{bf16,f16}; S is computed
//     transposed, S^T = K Q^T, so each lane owns ONE query (lane % 32) and 16 of
//     the 32 keys of a 32-key block: the row max needs one exchange between the
//     wave halves, the row sum none until the epilogue;
//   * O is accumulated transposed, O^T = V^T P^T: alpha is a per-lane scalar and P
//     is the MFMA B operand straight from the S registers (rounded to T);
//   * K and V tiles go global -> LDS by DMA (buffer_load ... lds, 16 B per lane),
//     with the buffer bound set to the head's remaining rows so that rows past Nk
//     read as zero without a branch; LDS rows are XOR-swizzled on 16-byte chunks
//     so that the K reads (ds_read_b128) and the V^T reads (ds_read_b64_tr_b16,
//     which hands each lane 4 consecutive keys of one column) hit 64 distinct
//     banks; the keys of V^T come out in exactly the order P has in registers;
//   * software pipeline: while the softmax of tile j and the P.V MFMAs of tile j
//     run, the S MFMAs of tile j+1 are issued; K and V have separate double
//     buffers with the next loads issued one tile ahead; one barrier per tile;
//   * exp is exp2 with scale*log2(e) folded into one FMA; the O rescale is skipped
//     when no row max of the wave moved (alpha = 1 exactly); the row sum l is taken
//     on the fp32 P before it is rounded for the MFMA (a sum of the rounded P would
//     put up to 2^-9 relative error into l, and so into L, on rows with few keys).
#pragma once

#include "fa_common.hpp"

namespace fa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <typename T>
struct Mfma16;

template <>
struct Mfma16<__bf16> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mfma16<_Float16> {
    typedef f16x8 vec;
    static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <int D>
struct Tile16 {
    static constexpr int BR = 128;              // query rows per workgroup
    static constexpr int BC = 64;               // keys per K/V tile
    static constexpr int NT = 256;              // threads per workgroup
    static constexpr int ROWB = D * 2;          // bytes per K/V row
    static constexpr int TILE = BC * ROWB;      // bytes per K or V tile
    static constexpr int LPW = TILE / 1024 / 4; // 1 KB DMA loads per wave per tile
    static constexpr int DC = D / 16;           // 16-wide d chunks of the S contraction
    static constexpr int DB = D / 32;           // 32-wide d blocks of O
    static constexpr int LDS = 4 * TILE;        // K[2] and V[2]
    static constexpr int K0 = 0, K1 = TILE, V0 = 2 * TILE, V1 = 3 * TILE;
    static_assert(LPW >= 1, "tile too small for the DMA staging");
};

// XOR applied to the 16-byte chunk index of LDS row `row` (bijective on 16
// consecutive rows; see the layout notes at the top of the file).
template <int D>
__device__ __forceinline__ int swz(int row)
{
    if constexpr (D == 128)
        return ((row & 3) << 2) | ((row >> 2) & 3);
    else
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Word 3 of a gfx9 buffer resource for untyped (raw) loads: 32-bit data format.
constexpr int kRsrcWord3 = 0x00020000;

// Buffer resource over rows [row0, nrows) of a [nrows, D] matrix: offsets past the
// end read as zero.
template <int D, typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const T* base, int row0, int nrows)
{
    const int n = nrows > row0 ? nrows - row0 : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base) + (size_t)row0 * D, 0,
                                             n * D * (int)sizeof(T), kRsrcWord3);
}

// DMA one K or V tile (rows [tile*BC, tile*BC + BC) of a head) into LDS: this wave's
// LPW 1-KB blocks starting at `dst`; lane i of each block lands at dst + 1024*blk + 16*i.
// A device function (not a lambda) so that the host pass never sees the builtin.
template <int D, typename T>
__device__ __forceinline__ void stage_tile(const T* head, int tile, int nrows, char* dst,
                                           const int* voff)
{
    using P = Tile16<D>;
    const __amdgpu_buffer_rsrc_t r = rows_rsrc<D>(head, tile * P::BC, nrows);
#pragma unroll
    for (int i = 0; i < P::LPW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + i * 1024), 16, voff[i], 0,
                                                 0, 0);
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_mfma16_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                          const T* __restrict__ V, T* __restrict__ O, float* __restrict__ LSE,
                          int Nq, int Nk, int n_qtiles, float c2)
{
    using P = Tile16<D>;
    using M = Mfma16<T>;
    using vec = typename M::vec;
    typedef T T4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(1024))) char smem[P::LDS];
    lds_char* const lds = (lds_char*)smem;
    const char* const sm = smem;

    // ---- which (batch*head, query tile) this workgroup owns
    const int logical = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int bh = logical / n_qtiles;
    int qt = logical - bh * n_qtiles;
    if (CAUSAL)
        qt = n_qtiles - 1 - qt;  // longest rows (most key tiles) are dispatched first
    const int q0 = qt * P::BR;

    const int tid = (int)threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ql = lane & 31;  // query column of this lane in the accumulators
    const int hh = lane >> 5;  // wave half
    const int qw0 = q0 + wave * 32;
    const int my_q = qw0 + ql;

    const T* Qh = Q + (size_t)bh * Nq * D;
    const T* Kh = K + (size_t)bh * Nk * D;
    const T* Vh = V + (size_t)bh * Nk * D;

    // ---- key tiles: the workgroup stages nkt of them; this wave computes n_w
    int nkt = (Nk + P::BC - 1) / P::BC;
    if (CAUSAL)
        nkt = min(nkt, (min(q0 + P::BR, Nq) - 1) / P::BC + 1);
    const bool wave_active = qw0 < Nq;
    int n_w = wave_active ? nkt : 0;
    if (CAUSAL && wave_active)
        n_w = min(nkt, min(qw0 + 31, Nq - 1) / P::BC + 1);

    // ---- DMA staging: per-lane byte offsets inside a tile (fixed for the kernel)
    int voff[P::LPW];
#pragma unroll
    for (int i = 0; i < P::LPW; ++i) {
        const int pos = (wave * P::LPW + i) * 1024 + lane * 16;
        const int row = pos / P::ROWB;
        const int pch = (pos % P::ROWB) / 16;
        voff[i] = row * P::ROWB + ((pch ^ swz<D>(row)) * 16);
    }
    auto stage = [&](const T* head, int tile, int lds_off) {
        stage_tile<D>(head, tile, Nk, smem + lds_off + wave * P::LPW * 1024, voff);
    };

    // ---- operand addresses inside a K / V buffer
    // K (A operand of S^T): lane reads K[32kb + ql][16c + 8hh .. +8]; kb adds 32 rows.
    int kaddr[P::DC];
#pragma unroll
    for (int c = 0; c < P::DC; ++c)
        kaddr[c] = ql * P::ROWB + (((2 * c + hh) ^ swz<D>(ql)) * 16);
    // V^T (A operand of O^T) by transpose reads: for (db, r) the 16-lane group g
    // reads rows 8r + 4h + j (j = 0..3) and columns 32db + 16(g%2) + 4a; 16-key
    // chunk cc adds 16 rows.
    int vaddr[P::DB][2];
    {
        const int g = lane >> 4, t = lane & 15;
        const int j = t >> 2, a = t & 3;
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int row = 8 * r + 4 * (g >> 1) + j;
                const int col = 32 * db + 16 * (g & 1) + 4 * a;
                vaddr[db][r] = row * P::ROWB + (((col >> 3) ^ swz<D>(row)) * 16) + (col & 7) * 2;
            }
    }

    // ---- prologue: tiles 0 and 1 in flight, Q fragment into registers
    if (0 < nkt) {
        stage(Kh, 0, P::K0);
        stage(Vh, 0, P::V0);
    }
    if (1 < nkt) {
        stage(Kh, 1, P::K1);
        stage(Vh, 1, P::V1);
    }
    // Q (B operand of S^T = K Q^T): lane supplies Q[my_q][16c + 8hh .. +8]
    vec qf[P::DC];
#pragma unroll
    for (int c = 0; c < P::DC; ++c) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (my_q < Nq)
            raw = *reinterpret_cast<const u32x4*>(Qh + (size_t)my_q * D + 16 * c + 8 * hh);
        qf[c] = __builtin_bit_cast(vec, raw);
    }

    // S^T of one key tile from the K buffer at byte offset kb_off
    auto scores = [&](int kb_off, f32x16* s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            s[kb] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < P::DC; ++c)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const vec a = *reinterpret_cast<const vec*>(sm + kb_off + kaddr[c] + kb * 32 * P::ROWB);
                s[kb] = M::mma(a, qf[c], s[kb]);
            }
    };

    // ---- running state: base-2 max, this half's partial sum, O^T accumulators
    f32x16 o[P::DB];
#pragma unroll
    for (int db = 0; db < P::DB; ++db)
        o[db] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    float m2 = neg_inf();
    float l = 0.f;

    // softmax of tile j (in s) and O^T += V_j^T P_j^T from the V buffer at vb_off
    auto softmax_pv = [&](int j, f32x16* s, int vb_off) {
        const int key0 = j * P::BC;
        const bool need_mask = (key0 + P::BC > Nk) || (CAUSAL && key0 + P::BC - 1 > qw0);
        if (need_mask) {
            // keys key0 + 4hh + off with off = 32kb + 8(r/4) + r%4 are visible iff off <= lim
            const int last = CAUSAL ? min(Nk - 1, my_q) : Nk - 1;
            const int lim = last - key0 - 4 * hh;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
                    if (off > lim)
                        s[kb][r] = neg_inf();
                }
        }
        // row max: 32 values in-lane, then the other wave half
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, swap_halves(mx));
        const float m_new = fmaxf(m2, mx * c2);  // c2 > 0: max commutes with the scale
        // a row that has seen no visible key yet keeps alpha = 1 and p = 0
        const bool none = (m_new == neg_inf());
        const float alpha = none ? 1.f : exp2_fast(m2 - m_new);
        const float mneg = none ? 0.f : -m_new;

        // P = 2^(s c2 - m_new) in fp32; the row sum is taken on these fp32 values
        // (four independent chains), then P is rounded to T and packed in the MFMA
        // B-operand order: chunk cc = 2kb + h holds registers 8h .. 8h+7 of block kb
        vec pb[4];
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = exp2_fast(fmaf(s[cc >> 1][8 * (cc & 1) + e], c2, mneg));
                rs[e & 3] += p;
                pb[cc][e] = (T)p;
            }
        l = l * alpha + ((rs[0] + rs[1]) + (rs[2] + rs[3]));
        // rescale O~ only if some row of the wave raised its max (else alpha == 1)
        if (__builtin_amdgcn_ballot_w64(m_new != m2) != 0) {
#pragma unroll
            for (int db = 0; db < P::DB; ++db)
                o[db] *= alpha;
        }
        m2 = m_new;

        // O^T += V^T P^T; the two transpose reads give keys 8r + 4h + 0..3 of chunk cc
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int db = 0; db < P::DB; ++db) {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(lds + (vb_off + cc * 16 * P::ROWB + vaddr[db][0])));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(lds + (vb_off + cc * 16 * P::ROWB + vaddr[db][1])));
                const vec a = __builtin_bit_cast(vec, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[db] = M::mma(a, pb[cc], o[db]);
            }
    };

    __syncthreads();  // waits for this wave's DMA (vmcnt) and publishes tiles 0, 1
    f32x16 sa[2], sb[2];
    if (0 < n_w)
        scores(P::K0, sa);
    __syncthreads();  // every wave has read K_0
    if (2 < nkt)
        stage(Kh, 2, P::K0);

    // one pipelined step: S of tile j+1 (from K buffer kn), softmax + P.V of tile j
    // (from V buffer vc); then publish the loads issued one step ago and issue the
    // next ones into the buffers this step has finished with
    auto step = [&](int j, f32x16* s_cur, f32x16* s_nxt, int kn, int vc) {
        if (j + 1 < n_w)
            scores(kn, s_nxt);
        if (j < n_w)
            softmax_pv(j, s_cur, vc);
        __syncthreads();
        if (j + 3 < nkt)
            stage(Kh, j + 3, kn);
        if (j + 2 < nkt)
            stage(Vh, j + 2, vc);
    };
    for (int j = 0; j < nkt; j += 2) {
        step(j, sa, sb, P::K1, P::V0);
        if (j + 1 < nkt)
            step(j + 1, sb, sa, P::K0, P::V1);
    }

    if (!wave_active)
        return;  // no barrier follows

    // ---- epilogue: O = O~ / l (rounded to T, nearest-even), L = ln2 * (m2 + log2 l)
    const float lt = l + swap_halves(l);
    if (my_q < Nq) {
        const float inv = 1.0f / lt;
        T* orow = O + ((size_t)bh * Nq + my_q) * D;
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                T4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = (T)(o[db][4 * a + e] * inv);
                *reinterpret_cast<T4*>(orow + 32 * db + 8 * a + 4 * hh) = w;
            }
        if (hh == 0)
            LSE[(size_t)bh * Nq + my_q] = (m2 + log2_fast(lt)) * kLn2;
    }
}

}  // namespace fa
