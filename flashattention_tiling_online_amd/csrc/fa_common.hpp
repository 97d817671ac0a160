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

// Check build (FA_DEBUG_FULL_BARRIER defined): every workgroup barrier of the kernels
// first waits for all of the wave's outstanding memory operations (global loads, DMA
// into LDS, LDS reads and writes).  Its outputs must equal the optimised build's bit
// for bit, which holds only if no kernel reads a buffer before the operation that
// fills it has completed, whatever the latencies.
#ifdef FA_DEBUG_FULL_BARRIER
constexpr bool kFullBarrier = true;
#else
constexpr bool kFullBarrier = false;
#endif

// The kernels' workgroup barrier (a full wait first in the check build).
__device__ __forceinline__ void wg_barrier()
{
    if (kFullBarrier)
        __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all zero
    __syncthreads();
}

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
    // caller mask (used by the masked instantiations only): bit-packed rows of
    // mask_w = ceil(Nk / 32) words, key k in bit k % 32 of word k / 32 (set = visible);
    // head bh = b * H + h reads the [Nq, mask_w] slice at mask + b * mask_sb + h * mask_sh
    // (strides in words, 0 where the mask is shared)
    const uint32_t* mask;
    int64_t mask_sb, mask_sh;
    int mask_w, H;
};

// The caller-mask slice of head bh (see FwdParams::mask).
template <typename Prm>
__device__ __forceinline__ const uint32_t* mask_slice(const Prm& prm, int bh)
{
    return prm.mask + (bh / prm.H) * prm.mask_sb + (bh % prm.H) * prm.mask_sh;
}

// Buffer resource over rows [row0, min(row0 + rows, Nq)) of a head's mask slice:
// words past the end read as zero (key k hidden).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mask_rsrc(const uint32_t* slice, int row0,
                                                           int rows, int Nq, int w)
{
    const int64_t n = min(row0 + rows, Nq) - row0;
    const int64_t bytes = (n > 0 ? n : 0) * (int64_t)w * 4;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(slice) + (size_t)row0 * w, 0,
                                             bytes < (1 << 30) ? (int)bytes : (1 << 30),
                                             0x00020000);
}

// Scores s[kb][r] of a 64-key tile whose keys, for lane half hh, sit at offsets
// 32 kb + 8 (r / 4) + 4 hh + r % 4 become -inf where the mask words w0 (keys 0-31 of
// the tile) and w1 (keys 32-63) have the key's bit clear.  Returns true when every
// key of every lane of the wave is visible (and nothing was changed).
__device__ __forceinline__ bool apply_mask_words(f32x16* s, uint32_t w0, uint32_t w1, int hh)
{
    const uint32_t a = w0 >> (4 * hh), b = w1 >> (4 * hh);
    const uint32_t lane_bits = 0x0F0F0F0Fu;  // this half's 16 keys of each word
    const bool all_mine = ((a & b & lane_bits) == lane_bits);
    if (__builtin_amdgcn_ballot_w64(!all_mine) == 0)
        return true;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const uint32_t w = kb ? b : a;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // all ones where the key is visible, zero where hidden (the score is copied
            // out of the vector before its bits are taken)
            const uint32_t keep = (uint32_t)(-(int32_t)((w >> (8 * (r >> 2) + (r & 3))) & 1u));
            const float x = s[kb][r];
            const uint32_t bits = __builtin_bit_cast(uint32_t, x);
            s[kb][r] = __builtin_bit_cast(float, (bits & keep) | (0xFF800000u & ~keep));
        }
    }
    return false;
}

// -inf as a float constant usable in device code
__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Exchange with the lane 32 positions away (the other half of a wave64).
// x of lanes 0-31 (lo) and of lanes 32-63 (hi) of the same lane pair (l, l ^ 32), both in
// every lane, from one v_permlane32_swap(x, x): its two results hold the low half of x
// in both halves and the high half in both halves.  A VALU exchange: unlike a shuffle
// (ds_bpermute) it does not queue behind other waves' LDS operand reads.  Combining lo
// and hi with a commutative operation gives every lane of the pair the same bits.
struct Halves {
    float lo, hi;
};
__device__ __forceinline__ Halves halves(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float half_max(float x)
{
    const Halves h = halves(x);
    return fmaxf(h.lo, h.hi);
}
__device__ __forceinline__ float half_sum(float x)
{
    const Halves h = halves(x);
    return h.lo + h.hi;
}

}  // namespace fa
