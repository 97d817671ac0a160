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

// Shader engines per XCD on gfx950 (8 CUs each).  Within an XCD the workgroups go to
// the engines round-robin in id order (rank j to engine j % 4); a workgroup waits
// for a free CU of its own engine, and the workgroups behind it wait with it.
constexpr int kSesPerXcd = 4;
// Items per XCD up to which causal grids are listed by weight (four rounds of the
// XCD's 32 CUs at one workgroup per CU).
constexpr int kSortedMax = 128;

// The work item of hardware workgroup `wg` of `n`, for a grid of (head, tile) items,
// n_tiles tiles per head: the head and the tile's rank.  Each XCD receives a
// contiguous range of the head-major order, so that the tiles of one head, which
// all stream the same K and V, share one L2.  Within an XCD the ranks are dealt to
// the shader engines in snake order (odd groups of four reversed), so that every
// engine receives a like share of a list ordered by weight.  With `heavy_first`
// (causal masks, where rank 0 is the heaviest tile), whole heads on the XCD and at
// most kSortedMax items on it, the list runs by rank across the XCD's heads: every
// engine then starts with its heaviest items, and each CU's later items pair up
// with its earlier ones (a CU that finishes a light item first takes the heaviest
// one left).  With more items per XCD the head-major order balances well enough by
// itself and keeps fewer heads' K and V in the XCD's L2 at a time.  A bijection
// from [0, n) onto the items for any n.
struct WorkItem {
    int head, rank;
};
__host__ __device__ __forceinline__ WorkItem work_item(int wg, int n, int n_tiles, bool heavy_first)
{
    const int per = n / kXcds;
    const int rem = n % kXcds;
    const int x = wg % kXcds;     // XCD this workgroup lands on
    const int j = wg / kXcds;     // its rank among that XCD's workgroups
    const int base = x * per + (x < rem ? x : rem);
    const int cnt = per + (x < rem ? 1 : 0);
    const int grp = j / kSesPerXcd, e = j % kSesPerXcd;
    const int r = ((grp & 1) && (grp + 1) * kSesPerXcd <= cnt) ? grp * kSesPerXcd + kSesPerXcd - 1 - e
                                                                : j;
    WorkItem w;
    if (heavy_first && cnt <= kSortedMax && base % n_tiles == 0 && cnt % n_tiles == 0) {
        const int m = cnt / n_tiles;  // heads on this XCD
        w.head = base / n_tiles + r % m;
        w.rank = r / m;
    } else {
        const int l = base + r;
        w.head = l / n_tiles;
        w.rank = l - w.head * n_tiles;
    }
    return w;
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
