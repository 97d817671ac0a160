// fa_merge.hpp — combine partial attention states computed over disjoint key ranges.
//
// Each part s holds, per query row, the normalised partial output O_s = O~_s / l_s
// and its log-sum-exp L_s = m_s + log l_s (fp32).  The blog page "Flash Attention"
// defines the (+) operator on (m, d, o~) states and shows it is associative and
// commutative, so the state over the union of the key ranges is the fold of the
// parts in any order.  In log-sum-exp form that fold is
//     L = M + log sum_s exp(L_s - M),   M = max_s L_s,
//     O = sum_s exp(L_s - L) * O_s,
// and a part whose range held no visible key (L_s = -inf, O_s = 0) is its
// identity.  A row with no visible key in any part keeps the identity: L = -inf and
// O = 0.
//
// Bound by memory traffic: per row it reads n_parts * (D + 1) fp32 values and
// writes D output elements and one fp32; one row is served by D/4 threads, one
// float4 each, so every part's row is read as one contiguous, coalesced segment.
#pragma once

#include "fa_common.hpp"

namespace fa {

template <typename T, int D>
struct Merge {
    static constexpr int TPR = D / 4;       // threads per row
    static constexpr int NT = 256;          // threads per workgroup
    static constexpr int RPB = NT / TPR;    // rows per workgroup
};

template <typename T, int D>
__global__ __launch_bounds__(256)
void fa_merge_kernel(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                     int n_parts, int64_t rows, T* __restrict__ O, float* __restrict__ LSE)
{
    using G = Merge<T, D>;
    typedef T T4 __attribute__((ext_vector_type(4)));
    const int64_t row = (int64_t)blockIdx.x * G::RPB + (int64_t)(threadIdx.x / G::TPR);
    const int t = (int)(threadIdx.x % G::TPR);
    if (row >= rows)
        return;

    // parts in groups of NG, each group's loads issued together (the fold is a
    // memory-bound stream: the loads, not the arithmetic, set its time)
    constexpr int NG = 8;
    float mx = neg_inf();
    for (int s0 = 0; s0 < n_parts; s0 += NG) {
        float l[NG];
#pragma unroll
        for (int u = 0; u < NG; ++u)
            l[u] = s0 + u < n_parts ? lse_part[(int64_t)(s0 + u) * rows + row] : neg_inf();
#pragma unroll
        for (int u = 0; u < NG; ++u)
            mx = fmaxf(mx, l[u]);
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (mx != neg_inf()) {
        for (int s0 = 0; s0 < n_parts; s0 += NG) {
            float l[NG];
            f32x4 v[NG];
#pragma unroll
            for (int u = 0; u < NG; ++u) {
                const bool in = s0 + u < n_parts;
                l[u] = in ? lse_part[(int64_t)(s0 + u) * rows + row] : neg_inf();
                v[u] = in ? *reinterpret_cast<const f32x4*>(o_part + ((int64_t)(s0 + u) * rows + row) * D + 4 * t)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < NG; ++u) {
                const float w = expf(l[u] - mx);  // 0 for an empty part or a missing one
                wsum += w;
                acc += w * v[u];
            }
        }
        acc *= 1.0f / wsum;
    }
    T4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        out[e] = (T)acc[e];
    *reinterpret_cast<T4*>(O + row * D + 4 * t) = out;
    if (t == 0)
        LSE[row] = mx != neg_inf() ? mx + logf(wsum) : neg_inf();
}

}  // namespace fa
