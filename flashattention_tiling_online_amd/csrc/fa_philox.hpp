// fa_philox.hpp — the random numbers of dropout on gfx950.
//
// Dropout acts on P after the softmax ("Flash Attention" blog page, Algorithm 2:
// P_dropped = dropout(P, p); Algorithm 4 regenerates the mask from the saved RNG
// state).  The generator is Philox4x32-10, written here from its published definition
// (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11):
// ten rounds of two 32x32 -> 64-bit products mixed with the other two counter words
// and the key, the key bumped by the Weyl constants between rounds.
//
// Element (q, k) of head bh uses key (seed low 32 bits, seed high 32 bits) and counter
// (k / 4, q / 4, bh, 0): one call covers the 4x4 block of queries 4(q/4).. and keys
// 4(k/4)..; its output word q % 4 holds the bytes of keys 4(k/4) + 0..3 (byte b =
// bits 8b..8b+7).  The element is dropped iff its byte is below the threshold t
// (drop probability t/256); kept values are scaled by 256/(256 - t).  A lane that
// owns one query and four consecutive keys reads one word of one call; a lane that
// owns one key and four consecutive queries reads one byte of each of the call's
// four words.
#pragma once

#include "fa_common.hpp"

namespace fa {

struct DropParams {
    uint32_t key0, key1;  // seed, low and high halves
    uint32_t t;           // drop iff byte < t
    float keep_scale;     // 256 / (256 - t)
};

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1)
{
    constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        const uint32_t hi0 = __umulhi(M0, c[0]), lo0 = M0 * c[0];
        const uint32_t hi1 = __umulhi(M1, c[2]), lo1 = M1 * c[2];
        c = u32x4{hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0};
    }
    return c;
}

// The four bytes of keys k4 .. k4+3 (k4 a multiple of 4) for query q of head bh.
__device__ __forceinline__ uint32_t drop_bytes_q(const DropParams& dp, int bh, int q, int k4)
{
    const u32x4 w = philox4x32_10(u32x4{(uint32_t)(k4 >> 2), (uint32_t)(q >> 2), (uint32_t)bh, 0u},
                                  dp.key0, dp.key1);
    const int s = q & 3;
    return s == 0 ? w[0] : s == 1 ? w[1] : s == 2 ? w[2] : w[3];
}

// The byte of key k for each of queries q4 .. q4+3 (q4 a multiple of 4), byte m of
// the result for query q4 + m.
__device__ __forceinline__ uint32_t drop_bytes_k(const DropParams& dp, int bh, int q4, int k)
{
    const u32x4 w = philox4x32_10(u32x4{(uint32_t)(k >> 2), (uint32_t)(q4 >> 2), (uint32_t)bh, 0u},
                                  dp.key0, dp.key1);
    const int sh = 8 * (k & 3);
    return ((w[0] >> sh) & 0xFFu) | (((w[1] >> sh) & 0xFFu) << 8) |
           (((w[2] >> sh) & 0xFFu) << 16) | (((w[3] >> sh) & 0xFFu) << 24);
}

// keep test of byte m of a word of four bytes
__device__ __forceinline__ bool drop_keep(uint32_t bytes, int m, uint32_t t)
{
    return ((bytes >> (8 * m)) & 0xFFu) >= t;
}

}  // namespace fa
