// fa_fwd_f32.hpp — fused attention forward for fp32 inputs on gfx950.
//
// Same recurrence and work decomposition as the bf16/fp16 kernel (the course page
// "05_flash_attention.py", flash_attention_forward; the blog page "Flash
// Attention" for the rescale of the unnormalised accumulator), but every operand
// stays fp32: both contractions use v_mfma_f32_32x32x2_f32, and P is fed to the
// second one without rounding.  This path exists for fp32 callers who need
// single-precision accuracy; it is simple rather than fast (single-buffered
// LDS, two barriers per tile).
//
// With a caller mask (blog page "Flash Attention", Algorithm 2: S_masked = mask(S)) the
// hidden scores become -inf from the mask words of the tile; a row that sees no key ends
// with O = 0 and L = -inf.
//
// Register layouts mirror the bf16 kernel: S^T = K Q^T and O^T = V^T P^T, so each
// lane owns one query.  With k = 2 per MFMA, lane half hh supplies one k index:
//   S:  A = K[key = 32kb + lane%32][d = 2c + hh],   B = Q[my_q][2c + hh]
//   PV: A = V[key(kb, t, hh)][d = 32db + lane%32],  B = P[my_q][key(kb, t, hh)]
// with key(kb, t, hh) = 32kb + 8(t/4) + 4hh + t%4 the key of accumulator register t.
// LDS strides: K rows D+2 floats (64 lanes hit 64 distinct banks), V rows D+8
// floats (the two wave halves read rows 4 apart, 32 banks apart).
#pragma once

#include "fa_common.hpp"

namespace fa {

template <int D>
struct TileF32 {
    static constexpr int BR = 128;
    static constexpr int BC = 64;
    static constexpr int NT = 256;
    static constexpr int KS = D + 2;
    static constexpr int VS = D + 8;
    static constexpr int CH = BC * D / 4 / NT;  // float4 chunks per thread per tensor
    static constexpr int DB = D / 32;
};

template <int D, bool CAUSAL, bool SPLIT, bool MASK = false>
__global__ __launch_bounds__(256)
void fa_fwd_f32_kernel(const FwdParams<float> prm)
{
    using P = TileF32<D>;
    __shared__ __attribute__((aligned(16))) float Ks[P::BC * P::KS];
    __shared__ __attribute__((aligned(16))) float Vs[P::BC * P::VS];
    const int Nq = prm.Nq, Nk = prm.Nk, n_qtiles = prm.n_qtiles;
    const float c2 = prm.c2;

    const WorkItem wi = work_item((int)blockIdx.x, (int)gridDim.x, n_qtiles, CAUSAL && !SPLIT);
    const int rest = wi.head;
    const int qt = CAUSAL ? n_qtiles - 1 - wi.rank : wi.rank;
    const int split = SPLIT ? rest % prm.n_splits : 0;
    const int bh = SPLIT ? rest / prm.n_splits : rest;
    const int q0 = qt * P::BR;

    const int tid = (int)threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ql = lane & 31;
    const int hh = lane >> 5;
    const int qw0 = q0 + wave * 32;
    const int my_q = qw0 + ql;

    // key range [kbeg, kbeg + Nks) of the head; key positions below are relative
    // to kbeg, and so are the queries' causal limits
    const int kbeg = SPLIT ? split * prm.split_tiles * P::BC : 0;
    const int Nks = SPLIT ? min(Nk - kbeg, prm.split_tiles * P::BC) : Nk;
    const int qkw0 = qw0 - kbeg;
    const int my_qk = my_q - kbeg;

    const float* Qh = prm.q + (size_t)bh * Nq * D;
    const float* Kh = prm.k + ((size_t)bh * Nk + kbeg) * D;
    const float* Vh = prm.v + ((size_t)bh * Nk + kbeg) * D;

    // caller mask: this lane's row of the head's mask slice
    static_assert(!(MASK && SPLIT), "the masked forward is not split");
    const __amdgpu_buffer_rsrc_t mrs = mask_rsrc(MASK ? mask_slice(prm, bh) : nullptr, q0, P::BR, Nq,
                                                 MASK ? prm.mask_w : 0);
    int mrow_off = 0;
    if (MASK)
        mrow_off = (my_q - q0) * prm.mask_w * 4;

    float qf[D / 2];
#pragma unroll
    for (int c = 0; c < D / 2; ++c)
        qf[c] = my_q < Nq ? Qh[(size_t)my_q * D + 2 * c + hh] : 0.f;

    int nkt = (Nks + P::BC - 1) / P::BC;
    if (CAUSAL) {
        const int qlast = min(q0 + P::BR, Nq) - 1 - kbeg;
        nkt = qlast < 0 ? 0 : min(nkt, qlast / P::BC + 1);
    }
    const bool wave_active = qw0 < Nq;
    const int qw_last = min(qw0 + 31, Nq - 1) - kbeg;  // may be negative: no key visible

    f32x16 o[P::DB];
#pragma unroll
    for (int db = 0; db < P::DB; ++db)
        o[db] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    float m2 = neg_inf();
    float l = 0.f;       // this half's row sum, current block of kSumBlock tiles
    float l_done = 0.f;  // completed blocks (bounds the drift of the fp32 sum)

    for (int j = 0; j < nkt; ++j) {
        const int key0 = j * P::BC;
        wg_barrier();  // previous tile fully consumed
#pragma unroll
        for (int i = 0; i < P::CH; ++i) {
            const int f = i * P::NT + tid;
            const int key = f / (D / 4);
            const int d4 = f % (D / 4);
            const int gk = key0 + key;
            f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (gk < Nks) {
                kv = *reinterpret_cast<const f32x4*>(Kh + (size_t)gk * D + 4 * d4);
                vv = *reinterpret_cast<const f32x4*>(Vh + (size_t)gk * D + 4 * d4);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Ks[key * P::KS + 4 * d4 + e] = kv[e];
            *reinterpret_cast<f32x4*>(Vs + key * P::VS + 4 * d4) = vv;
        }
        wg_barrier();

        if (!wave_active || (CAUSAL && key0 > qw_last))
            continue;

        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < D / 2; ++c)
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[(32 * kb + ql) * P::KS + 2 * c + hh],
                                                             qf[c], s[kb], 0, 0, 0);
        }

        if (MASK)
            apply_mask_words(s, __builtin_amdgcn_raw_buffer_load_b32(mrs, mrow_off + 8 * j, 0, 0),
                             __builtin_amdgcn_raw_buffer_load_b32(mrs, mrow_off + 8 * j + 4, 0, 0),
                             hh);
        const bool need_mask = (key0 + P::BC > Nks) || (CAUSAL && key0 + P::BC - 1 > qkw0);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key >= Nks || (CAUSAL && key > my_qk))
                        s[kb][r] = neg_inf();
                }
        }

        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx = fmaxf(mx, s[kb][r]);
        mx = half_max(mx);
        const float m_new = fmaxf(m2, mx * c2);
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
        l_done *= alpha;
        if ((j & (kSumBlock - 1)) == kSumBlock - 1) {
            l_done += l;
            l = 0.f;
        }
        m2 = m_new;
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
            o[db] *= alpha;

#pragma unroll
        for (int db = 0; db < P::DB; ++db)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const int key = 32 * kb + 8 * (t >> 2) + 4 * hh + (t & 3);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * P::VS + 32 * db + ql],
                                                                 s[kb][t], o[db], 0, 0, 0);
                }
    }

    if (!wave_active)
        return;
    // split: a row that saw no key of its range leaves the merge identity
    // (L = -inf, O = 0)
    const float lsum = l_done + l;
    const float lt = half_sum(lsum);
    if (my_q < Nq) {
        const size_t row = SPLIT ? ((size_t)split * prm.bh_count + bh) * Nq + my_q
                                 : (size_t)bh * Nq + my_q;
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        float* orow = (SPLIT ? prm.o_part : prm.o) + row * D;
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = o[db][4 * a + e] * inv;
                *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * a + 4 * hh) = w;
            }
        if (hh == 0)
            (SPLIT ? prm.lse_part : prm.lse)[row] =
                lt > 0.f ? (m2 + log2_fast(lt)) * kLn2 : neg_inf();
    }
}

}  // namespace fa
