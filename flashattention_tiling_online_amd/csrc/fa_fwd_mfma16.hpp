// fa_fwd_mfma16.hpp — fused attention forward for bf16 / fp16 inputs on gfx950.
//
// The algorithm is the query-outer, key-inner online-softmax recurrence of the
// course page "05_flash_attention.py" (flash_attention_forward): per query tile
// m = -inf, l = 0, O~ = 0; for each key/value tile, left to right:
//     S = Q_i K_j^T * scale,  m_new = max(m, rowmax S),  P = exp(S - m_new),
//     alpha = exp(m - m_new), l = alpha l + rowsum P, O~ = alpha O~ + P V_j;
// at the end O = O~ / l and L = m + log l.  The rescale of the unnormalised O~
// uses exp(m_old - m_new) alone, as in the "Flash Attention" blog page's (+)
// operator on (m, d, o~).  Key tiles wholly in the causal future are skipped and
// only tiles that straddle the diagonal (or the ragged end of the keys) are masked
// (course page, causal branch of flash_attention_forward).
//
// gfx950 mapping (not taken from the pages, which describe an NVIDIA design):
//   * workgroup = 4 wave64s = 128 query rows; wave w owns rows [32w, 32w+32);
//   * both contractions run on v_mfma_f32_32x32x16_{bf16,f16};
//   * S is computed transposed, S^T = K Q^T, so that in the accumulator each lane
//     owns ONE query (lane % 32) and 16 of the 32 keys of a 32-key block; the row
//     max needs one exchange between the two wave halves, and the row sum none
//     until the epilogue (each half keeps a partial l; both see the same alpha);
//   * O is accumulated transposed too, O^T = V^T P^T, so alpha is a per-lane
//     scalar and P feeds the MFMA B operand straight from the S registers;
//   * the key order inside the P.V contraction is free, so V is stored transposed
//     in LDS with its keys permuted to the order P already has in registers
//     (the transpose happens in registers while staging a tile);
//   * exp is exp2 with scale*log2(e) folded into one FMA: p = 2^(s*c - m2);
//   * K and V^T tiles are double-buffered in LDS with register prefetch of the
//     next tile, one barrier per tile; rows are padded by 8 elements so that the
//     16-byte LDS reads of 16 consecutive lanes hit distinct banks.
#pragma once

#include "fa_common.hpp"

namespace fa {

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
    static constexpr int KS = D + 8;            // K row stride in LDS (elements)
    static constexpr int VS = BC + 8;           // V^T row stride in LDS (elements)
    static constexpr int K_ELEMS = BC * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
    static constexpr int KCH = BC * D / 8 / NT; // 16-byte K chunks staged per thread
    static constexpr int VBLK = BC * D / 32;    // (8 keys x 4 dims) V blocks per tile
    static constexpr int DC = D / 16;           // 16-wide d chunks of the S contraction
    static constexpr int DB = D / 32;           // 32-wide d blocks of O
    static_assert(KCH >= 1 && VBLK <= NT, "tile does not fit the staging scheme");
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_mfma16_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                          const T* __restrict__ V, T* __restrict__ O, float* __restrict__ LSE,
                          int Nq, int Nk, int n_qtiles, float c2)
{
    using P = Tile16<D>;
    using vec = typename Mfma16<T>::vec;
    typedef T T4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) T smem[2 * P::BUF_ELEMS];

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

    // ---- Q fragment, held for the whole loop: B operand of S^T = K Q^T.
    // Lane (ql, hh) supplies Q[my_q][16c + 8hh .. +8) for d chunk c.
    vec qf[P::DC];
#pragma unroll
    for (int c = 0; c < P::DC; ++c) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (my_q < Nq)
            raw = *reinterpret_cast<const u32x4*>(Qh + (size_t)my_q * D + 16 * c + 8 * hh);
        qf[c] = __builtin_bit_cast(vec, raw);
    }

    // ---- key tiles this workgroup visits (causal: none past its last query)
    int nkt = (Nk + P::BC - 1) / P::BC;
    if (CAUSAL) {
        const int qlast = min(q0 + P::BR, Nq) - 1;
        nkt = min(nkt, qlast / P::BC + 1);
    }
    const bool wave_active = qw0 < Nq;
    const int qw_last = min(qw0 + 31, Nq - 1);

    // ---- staging registers (next tile in flight while the current one computes)
    u32x4 kreg[P::KCH];
    u32x2 vreg[8];
    // V block of this thread: 8 keys x 4 dims.  Group g = 2*cp + hp covers the keys
    // {16cp + 4hp + 0..3, 16cp + 8 + 4hp + 0..3}: exactly the 8 keys that wave half hp
    // feeds, in this order, to the MFMA of 16-key chunk cp.
    const bool v_owner = tid < P::VBLK;
    const int v_d4 = tid % (D / 4);
    const int v_g = tid / (D / 4);
    const int v_cp = v_g >> 1;
    const int v_hp = v_g & 1;

    auto load_tile = [&](int j) {
        const int key0 = j * P::BC;
#pragma unroll
        for (int i = 0; i < P::KCH; ++i) {
            const int f = i * P::NT + tid;
            const int key = f / (D / 8);
            const int dc = f % (D / 8);
            const int gk = key0 + key;
            kreg[i] = gk < Nk ? *reinterpret_cast<const u32x4*>(Kh + (size_t)gk * D + dc * 8)
                              : u32x4{0u, 0u, 0u, 0u};
        }
        if (v_owner) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int key = 16 * v_cp + 8 * (jj >> 2) + 4 * v_hp + (jj & 3);
                const int gk = key0 + key;
                vreg[jj] = gk < Nk ? *reinterpret_cast<const u32x2*>(Vh + (size_t)gk * D + 4 * v_d4)
                                   : u32x2{0u, 0u};
            }
        }
    };

    auto store_tile = [&](T* Ks, T* Vt) {
#pragma unroll
        for (int i = 0; i < P::KCH; ++i) {
            const int f = i * P::NT + tid;
            const int key = f / (D / 8);
            const int dc = f % (D / 8);
            *reinterpret_cast<u32x4*>(Ks + key * P::KS + dc * 8) = kreg[i];
        }
        if (v_owner) {
            // transpose 8 keys x 4 dims into 4 rows of V^T, 8 keys each
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u32x4 w;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t a = (e < 2) ? vreg[2 * p].x : vreg[2 * p].y;
                    const uint32_t b = (e < 2) ? vreg[2 * p + 1].x : vreg[2 * p + 1].y;
                    w[p] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u))
                                   : ((a & 0xffffu) | (b << 16));
                }
                *reinterpret_cast<u32x4*>(Vt + (4 * v_d4 + e) * P::VS + 16 * v_cp + 8 * v_hp) = w;
            }
        }
    };

    // ---- running state: base-2 max, this half's partial sum, O^T accumulators
    f32x16 o[P::DB];
#pragma unroll
    for (int db = 0; db < P::DB; ++db)
        o[db] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    float m2 = neg_inf();
    float l = 0.f;

    load_tile(0);
    for (int j = 0; j < nkt; ++j) {
        T* Ks = smem + (j & 1) * P::BUF_ELEMS;
        T* Vt = Ks + P::K_ELEMS;
        store_tile(Ks, Vt);
        __syncthreads();
        if (j + 1 < nkt)
            load_tile(j + 1);

        const int key0 = j * P::BC;
        if (!wave_active)
            continue;
        if (CAUSAL && key0 > qw_last)
            continue;  // every key of the tile is in the future of every row of this wave

        // S^T for the two 32-key blocks: s[kb][r] = S[my_q][key0 + 32kb + 8(r/4) + 4hh + r%4]
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < P::DC; ++c) {
                const vec a = *reinterpret_cast<const vec*>(Ks + (32 * kb + ql) * P::KS + 16 * c + 8 * hh);
                s[kb] = Mfma16<T>::mma(a, qf[c], s[kb]);
            }
        }

        // mask: keys past the end, and (causal) keys after the query
        const bool need_mask = (key0 + P::BC > Nk) || (CAUSAL && key0 + P::BC - 1 > qw0);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key >= Nk || (CAUSAL && key > my_q))
                        s[kb][r] = neg_inf();
                }
        }

        // row max over the tile: 32 values in-lane, then the other wave half
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

        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = exp2_fast(fmaf(s[kb][r], c2, mneg));
                s[kb][r] = p;
                rs += p;
            }
        l = l * alpha + rs;
        m2 = m_new;
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
            o[db] *= alpha;

        // P as the MFMA B operand: chunk cc = 2kb + h holds registers 8h .. 8h+7 of block kb
        vec pb[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pb[cc][e] = (T)s[cc >> 1][8 * (cc & 1) + e];

        // O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const vec a = *reinterpret_cast<const vec*>(Vt + (32 * db + ql) * P::VS + 16 * cc + 8 * hh);
                o[db] = Mfma16<T>::mma(a, pb[cc], o[db]);
            }
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
