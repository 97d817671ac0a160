// fa_common.hpp — device-side helpers shared by the gfx950 attention kernels.
//
// Work decomposition: one workgroup per (batch*head, query tile), as in the
// course page "05_flash_attention.py" (flash_attention_forward: each query block
// is owned by one thread block and its state stays on chip) — or, split along the
// keys, per (batch*head, key range, query tile), each range leaving a partial
// (O, L) state that the merge kernel folds with the (+) operator of the blog page
// "Flash Attention" in its log-sum-exp form.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309417f;
// key tiles per block of the forward kernels' row sums (a power of two)
constexpr int kSumBlock = 64;

// Number of XCDs (accelerator complex dies) on gfx950.  Consecutive workgroup ids
// are dispatched round-robin over them, and each has its own L2.
constexpr int kXcds = 8;

// Map the hardware workgroup id to a logical tile id so that the logical ids an
// XCD receives are contiguous.  Logical ids are ordered head-major, so the query
// tiles of one head — which all stream the same K and V — share one XCD's L2.
// A bijection on [0, n) for any n.
__device__ __forceinline__ int xcd_remap(int wg, int n)
{
    const int per = n / kXcds;
    const int rem = n % kXcds;
    const int x = wg % kXcds;     // XCD this workgroup lands on
    const int j = wg / kXcds;     // its rank among that XCD's workgroups
    return x * per + (x < rem ? x : rem) + j;
}

// Arguments of one forward launch.  q, o: [bh_count, Nq, D]; k, v: [bh_count, Nk, D];
// lse: [bh_count, Nq].  With key splits (n_splits > 1) the workgroup for split s
// covers key tiles [s * split_tiles, (s + 1) * split_tiles) and writes fp32 partials
// o_part [n_splits, bh_count, Nq, D] and lse_part [n_splits, bh_count, Nq] instead
// of o and lse.
template <typename T>
struct FwdParams {
    const T* q;
    const T* k;
    const T* v;
    T* o;
    float* lse;
    float* o_part;
    float* lse_part;
    int Nq, Nk, n_qtiles, bh_count, n_splits, split_tiles;
    float c2;  // scale * log2(e)
    // dropout on P (used by the dropout instantiations only): seed halves, byte
    // threshold and keep scale, as in fa_philox.hpp
    uint32_t drop_key0, drop_key1, drop_t;
    float drop_keep_scale;
};

// -inf as a float constant usable in device code
__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Exchange with the lane 32 positions away (the other half of a wave64).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

}  // namespace fa
