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

// a ^ b ^ c in one instruction (gfx950's three-input bitwise op; 0x96 is the truth
// table of the three-way exclusive or)
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c)
{
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

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
        // both halves of each 32 x 32 -> 64-bit product from one multiply
        const uint64_t p0 = (uint64_t)M0 * c[0];
        const uint64_t p1 = (uint64_t)M1 * c[2];
        c = u32x4{xor3((uint32_t)(p1 >> 32), c[1], k0), (uint32_t)p1,
                  xor3((uint32_t)(p0 >> 32), c[3], k1), (uint32_t)p0};
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

// ---- sharing one call between the four lanes of a quad.  A call covers 4 queries x
// 4 keys; when the four lanes of a quad (lanes 4a .. 4a+3, all active) own four
// consecutive queries (or keys), each lane computes one call of four and the quad
// exchanges the words with DPP, instead of every lane computing all four calls.

// value of lane s ^ 1 / s ^ 2 of the quad
__device__ __forceinline__ uint32_t quad_xor1(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
}

// 4 x 4 transpose across a quad: lane s holds a[i] = M[s][i] and ends with a[i] = M[i][s]
// (two butterfly stages; in each, a lane trades the entries whose index bit differs
// from its own lane bit for its partner's mirrored entries).
__device__ __forceinline__ void quad_transpose(uint32_t* a, int s)
{
    const bool odd = (s & 1) != 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t r = quad_xor1(odd ? a[2 * k] : a[2 * k + 1]);
        if (odd)
            a[2 * k] = r;
        else
            a[2 * k + 1] = r;
    }
    const bool up = (s & 2) != 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t r = quad_xor2(up ? a[k] : a[k + 2]);
        if (up)
            a[k] = r;
        else
            a[k + 2] = r;
    }
}

// Lane = query q (queries 4(q/4) + 0..3 on the lanes of the quad): words[G] (G = 0..7)
// = the bytes of keys kbase + 8G + 0..3 for q, as drop_bytes_q(dp, bh, q, kbase + 8G);
// kbase a multiple of 4.  Two calls per lane.
__device__ __forceinline__ void drop_words_q8(const DropParams& dp, int bh, int q, int kbase,
                                              uint32_t* words)
{
    const int s = q & 3;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int g = s + 4 * half;
        const u32x4 w = philox4x32_10(
            u32x4{(uint32_t)((kbase + 8 * g) >> 2), (uint32_t)(q >> 2), (uint32_t)bh, 0u}, dp.key0,
            dp.key1);
        uint32_t a[4] = {w[0], w[1], w[2], w[3]};
        quad_transpose(a, s);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            words[4 * half + i] = a[i];
    }
}

// Lane = key k (keys 4(k/4) + 0..3 on the lanes of the quad): words[g] (g = 0..3) =
// the byte of key k for queries qbase + 8g + 0..3 (byte m for query qbase + 8g + m),
// as drop_bytes_k(dp, bh, qbase + 8g, k); qbase a multiple of 4.  One call per lane.
__device__ __forceinline__ void drop_words_k4(const DropParams& dp, int bh, int qbase, int k,
                                              uint32_t* words)
{
    const int s = k & 3;
    const u32x4 w = philox4x32_10(
        u32x4{(uint32_t)(k >> 2), (uint32_t)((qbase + 8 * s) >> 2), (uint32_t)bh, 0u}, dp.key0,
        dp.key1);
    // byte transpose inside the lane: a[b] = byte b (key 4(k/4) + b) of words 0..3
#pragma unroll
    for (int b = 0; b < 4; ++b)
        words[b] = ((w[0] >> (8 * b)) & 0xFFu) | (((w[1] >> (8 * b)) & 0xFFu) << 8) |
                   (((w[2] >> (8 * b)) & 0xFFu) << 16) | (((w[3] >> (8 * b)) & 0xFFu) << 24);
    // words[b] now belongs to (group s, key b); the quad transpose hands lane s' the
    // words of (group g, key s') for g = 0..3
    quad_transpose(words, s);
}

// keep test of byte m of a word of four bytes
__device__ __forceinline__ bool drop_keep(uint32_t bytes, int m, uint32_t t)
{
    return ((bytes >> (8 * m)) & 0xFFu) >= t;
}

// Dropout on four 16-bit values packed in two words (pairs[0] holds values 0, 1 in its
// low and high halves, pairs[1] values 2, 3), value m decided by byte m of `bytes`:
// zeroed iff the byte is below t (0 <= t <= 256).  Works on the packed words: each
// byte pair is spread into two 16-bit lanes, byte - t is negative exactly for the
// dropped values, and its sign, replicated over the lane, clears them.
__device__ __forceinline__ void drop_zero_pairs(uint32_t bytes, uint32_t* pairs, uint32_t t)
{
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    const s16x2 tt = {(short)t, (short)t};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // bytes 2h, 2h + 1 into the low bytes of the two 16-bit lanes (selector 0x0C: zero)
        const uint32_t x = __builtin_amdgcn_perm(0u, bytes, h ? 0x0C030C02u : 0x0C010C00u);
        const s16x2 d = __builtin_bit_cast(s16x2, x) - tt;
        const s16x2 drop = d >> (short)15;  // 0xFFFF where the byte is below t
        pairs[h] &= ~__builtin_bit_cast(uint32_t, drop);
    }
}

}  // namespace fa
