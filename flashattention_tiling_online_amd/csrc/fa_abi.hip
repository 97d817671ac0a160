// fa_abi.hip — the C-ABI of libfa.so: argument validation and kernel dispatch.
//
// Declared in include/fa.h.  Every argument error is returned before any HIP call;
// the kernel is enqueued with hipLaunchKernel so that its own launch status is
// returned (no sticky error from earlier, unrelated calls is consumed).
#include <math.h>
#include <stdint.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/fa.h"
#include "fa_bwd.hpp"
#include "fa_fwd_f32.hpp"
#include "fa_fwd_mfma16.hpp"
#include "fa_fwd_pp.hpp"
#include "fa_merge.hpp"

namespace {

constexpr int kKeyTile = 64;     // keys per tile in every kernel (the split granularity)
constexpr int kMaxSplits = 256;  // most key ranges fa_fwd_split accepts
constexpr int64_t kAlign = 256;  // alignment of the partial-L block in the workspace
// d = 64 forward: key groups per workgroup when the grid of 128-row workgroups would
// leave CUs without one (kSmallGridWgs or fewer workgroups)
constexpr int kKeyGroups = 4;
constexpr int64_t kSmallGridWgs = 256;

struct Launch {
    const void* fn;  // device function address
    int rows;        // query rows per workgroup
    int threads;     // threads per workgroup
};

template <typename T, int D, bool C, bool S>
Launch mfma16()
{
    return Launch{reinterpret_cast<const void*>(&fa::fa_fwd_mfma16_kernel<T, D, C, S>),
                  fa::Tile16<D>::BR, fa::Tile16<D>::NT};
}

// d = 64 with KG key groups per workgroup (for grids too small to fill the chip)
template <typename T, bool C>
Launch mfma16_kg()
{
    return Launch{reinterpret_cast<const void*>(
                      &fa::fa_fwd_mfma16_kernel<T, 64, C, false, false, false, kKeyGroups>),
                  fa::Tile16<64, kKeyGroups>::BR, fa::Tile16<64, kKeyGroups>::NT};
}

template <int D, bool C, bool S>
Launch f32()
{
    return Launch{reinterpret_cast<const void*>(&fa::fa_fwd_f32_kernel<D, C, S>),
                  fa::TileF32<D>::BR, fa::TileF32<D>::NT};
}

template <typename T, bool C, bool S>
Launch pp()
{
    return Launch{reinterpret_cast<const void*>(&fa::fa_fwd_pp_kernel<T, C, S>), fa::TilePP::BR,
                  fa::TilePP::NT};
}

// d = 128: the phase-alternating kernel (with or without key splits); d = 64:
// fa_fwd_mfma16
template <typename T, bool S>
Launch fwd16_of(int64_t d, bool c)
{
    if (d == 128)
        return c ? pp<T, true, S>() : pp<T, false, S>();
    return c ? mfma16<T, 64, true, S>() : mfma16<T, 64, false, S>();
}

template <bool S>
Launch f32_of(int64_t d, bool c)
{
    return d == 128 ? (c ? f32<128, true, S>() : f32<128, false, S>())
                    : (c ? f32<64, true, S>() : f32<64, false, S>());
}

bool pick(fa_dtype_t dtype, int64_t d, int causal, bool split, Launch* out)
{
    const bool c = causal != 0;
    if (d != 64 && d != 128)
        return false;
    switch (dtype) {
    case FA_DTYPE_BF16:
        *out = split ? fwd16_of<__bf16, true>(d, c) : fwd16_of<__bf16, false>(d, c);
        return true;
    case FA_DTYPE_F16:
        *out = split ? fwd16_of<_Float16, true>(d, c) : fwd16_of<_Float16, false>(d, c);
        return true;
    case FA_DTYPE_F32:
        *out = split ? f32_of<true>(d, c) : f32_of<false>(d, c);
        return true;
    }
    return false;
}

// the forward kernel with dropout on P (16-bit inputs, unsplit): d = 128 on the
// phase-alternating kernel, d = 64 on fa_fwd_mfma16
template <typename T>
Launch fwd16_drop(int64_t d, bool c)
{
    auto one = [](const void* fn, int rows, int threads) { return Launch{fn, rows, threads}; };
    if (d == 128)
        return c ? one(reinterpret_cast<const void*>(&fa::fa_fwd_pp_kernel<T, true, false, true>),
                       fa::TilePP::BR, fa::TilePP::NT)
                 : one(reinterpret_cast<const void*>(&fa::fa_fwd_pp_kernel<T, false, false, true>),
                       fa::TilePP::BR, fa::TilePP::NT);
    return c ? one(reinterpret_cast<const void*>(&fa::fa_fwd_mfma16_kernel<T, 64, true, false, true>),
                   fa::Tile16<64>::BR, fa::Tile16<64>::NT)
             : one(reinterpret_cast<const void*>(&fa::fa_fwd_mfma16_kernel<T, 64, false, false, true>),
                   fa::Tile16<64>::BR, fa::Tile16<64>::NT);
}

// the forward kernel with a caller mask (unsplit): d = 128 on the phase-alternating
// kernel, d = 64 on fa_fwd_mfma16, fp32 on fa_fwd_f32
template <typename T>
Launch fwd16_mask(int64_t d, bool c)
{
    if (d == 128)
        return c ? Launch{reinterpret_cast<const void*>(&fa::fa_fwd_pp_kernel<T, true, false, false, true>),
                          fa::TilePP::BR, fa::TilePP::NT}
                 : Launch{reinterpret_cast<const void*>(&fa::fa_fwd_pp_kernel<T, false, false, false, true>),
                          fa::TilePP::BR, fa::TilePP::NT};
    return c ? Launch{reinterpret_cast<const void*>(&fa::fa_fwd_mfma16_kernel<T, 64, true, false, false, true>),
                      fa::Tile16<64>::BR, fa::Tile16<64>::NT}
             : Launch{reinterpret_cast<const void*>(&fa::fa_fwd_mfma16_kernel<T, 64, false, false, false, true>),
                      fa::Tile16<64>::BR, fa::Tile16<64>::NT};
}

template <int D>
Launch f32_mask(bool c)
{
    return c ? Launch{reinterpret_cast<const void*>(&fa::fa_fwd_f32_kernel<D, true, false, true>),
                      fa::TileF32<D>::BR, fa::TileF32<D>::NT}
             : Launch{reinterpret_cast<const void*>(&fa::fa_fwd_f32_kernel<D, false, false, true>),
                      fa::TileF32<D>::BR, fa::TileF32<D>::NT};
}

Launch fwd_mask_of(fa_dtype_t dtype, int64_t d, bool c)
{
    switch (dtype) {
    case FA_DTYPE_BF16: return fwd16_mask<__bf16>(d, c);
    case FA_DTYPE_F16: return fwd16_mask<_Float16>(d, c);
    default: return d == 128 ? f32_mask<128>(c) : f32_mask<64>(c);
    }
}

// the byte threshold of a drop probability: t = round(256 p); -1 outside [0, 1) or
// beyond 255
int drop_threshold(float p)
{
    if (!(p >= 0.0f) || !(p < 1.0f))
        return -1;
    const long t = lrintf(p * 256.0f);
    return t > 255 ? -1 : (int)t;
}

// Workgroups of the forward kernel that one CU holds at once (register and LDS
// budgets of the kernels above): used only by fa_split_hint.
int wgs_per_cu(fa_dtype_t dtype, int64_t d) { return d == 64 ? 2 : 1; }

const void* merge_fn(fa_dtype_t dtype, int64_t d)
{
    switch (dtype) {
    case FA_DTYPE_BF16:
        return d == 128 ? reinterpret_cast<const void*>(&fa::fa_merge_kernel<__bf16, 128>)
                        : reinterpret_cast<const void*>(&fa::fa_merge_kernel<__bf16, 64>);
    case FA_DTYPE_F16:
        return d == 128 ? reinterpret_cast<const void*>(&fa::fa_merge_kernel<_Float16, 128>)
                        : reinterpret_cast<const void*>(&fa::fa_merge_kernel<_Float16, 64>);
    case FA_DTYPE_F32:
        return d == 128 ? reinterpret_cast<const void*>(&fa::fa_merge_kernel<float, 128>)
                        : reinterpret_cast<const void*>(&fa::fa_merge_kernel<float, 64>);
    }
    return nullptr;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a * b for non-negative a and b, INT64_MAX when the product does not fit: size checks
// compare it with their limits, so an argument whose product would wrap is refused
int64_t mul_sat(int64_t a, int64_t b)
{
    int64_t r;
    return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

bool valid_dtype(fa_dtype_t dtype)
{
    return dtype == FA_DTYPE_F32 || dtype == FA_DTYPE_F16 || dtype == FA_DTYPE_BF16;
}

// Checks shared by fa_fwd and fa_fwd_split, in the documented order; *empty is set
// when there is nothing to compute.
fa_status_t check_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                      int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                      fa_dtype_t dtype, bool split, Launch* L, bool* empty)
{
    *empty = false;
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
        return FA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype))
        return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1)
        return FA_ERR_INVALID_ARG;
    if (!(scale > 0.0f) || !isfinite(scale))
        return FA_ERR_INVALID_ARG;
    if (!pick(dtype, d, causal, split, L))
        return FA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || Nq == 0) {
        *empty = true;  // nothing to compute: no buffer is touched, pointers may be null
        return FA_OK;
    }
    if (!q || !k || !v || !o || !lse)
        return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(lse, 4))
        return FA_ERR_INVALID_ARG;
    if (Nk == 0)
        return FA_ERR_INVALID_ARG;  // softmax over an empty key set is undefined

    // size limits: in-head offsets are 32-bit, the grid is 1-D
    const int64_t lim = INT32_MAX;
    if (mul_sat(Nq, d) > lim || mul_sat(Nk, d) > lim || mul_sat(B, H) > lim)
        return FA_ERR_INVALID_ARG;
    const int64_t n_qtiles = (Nq + L->rows - 1) / L->rows;
    if (n_qtiles * B * H > lim)
        return FA_ERR_INVALID_ARG;
    return FA_OK;
}

// exp(x) = 2^(x * log2 e): fold log2(e) into the scale once, in double
float scale_log2e(float scale) { return (float)((double)scale * 1.4426950408889634074); }

// dropout on P: byte threshold t (drop probability t / 256) and the 64-bit seed
struct Dropout {
    uint32_t t;
    uint64_t seed;
};

// a caller mask: the words, their strides per batch and head (0 = shared), the words
// per row and the head count that splits b * H + h
struct MaskArg {
    const uint32_t* words;
    int64_t sb, sh;
    int w, H;
};

template <typename T>
hipError_t launch_fwd(const Launch& L, const void* q, const void* k, const void* v, void* o,
                      float* lse, float* o_part, float* lse_part, int64_t BH, int64_t Nq,
                      int64_t Nk, int n_splits, int split_tiles, float scale, hipStream_t stream,
                      const Dropout* drop = nullptr, const MaskArg* mask = nullptr)
{
    fa::FwdParams<T> prm;
    prm.mask = mask ? mask->words : nullptr;
    prm.mask_sb = mask ? mask->sb : 0;
    prm.mask_sh = mask ? mask->sh : 0;
    prm.mask_w = mask ? mask->w : 0;
    prm.H = mask ? mask->H : 1;
    prm.drop_key0 = drop ? (uint32_t)drop->seed : 0u;
    prm.drop_key1 = drop ? (uint32_t)(drop->seed >> 32) : 0u;
    prm.drop_t = drop ? drop->t : 0u;
    prm.drop_keep_scale = drop ? (float)(256.0 / (256.0 - (double)drop->t)) : 1.0f;
    prm.q = static_cast<const T*>(q);
    prm.k = static_cast<const T*>(k);
    prm.v = static_cast<const T*>(v);
    prm.o = static_cast<T*>(o);
    prm.lse = lse;
    prm.o_part = o_part;
    prm.lse_part = lse_part;
    prm.Nq = (int)Nq;
    prm.Nk = (int)Nk;
    prm.n_qtiles = (int)((Nq + L.rows - 1) / L.rows);
    prm.bh_count = (int)BH;
    prm.n_splits = n_splits;
    prm.split_tiles = split_tiles;
    prm.c2 = scale_log2e(scale);
    void* args[] = {(void*)&prm};
    const int64_t grid = (int64_t)prm.n_qtiles * BH * n_splits;
    return hipLaunchKernel(L.fn, dim3((unsigned)grid), dim3((unsigned)L.threads), args, 0, stream);
}

hipError_t launch_fwd_any(fa_dtype_t dtype, const Launch& L, const void* q, const void* k,
                          const void* v, void* o, float* lse, float* o_part, float* lse_part,
                          int64_t BH, int64_t Nq, int64_t Nk, int n_splits, int split_tiles,
                          float scale, hipStream_t stream, const Dropout* drop = nullptr,
                          const MaskArg* mask = nullptr)
{
    switch (dtype) {
    case FA_DTYPE_BF16:
        return launch_fwd<__bf16>(L, q, k, v, o, lse, o_part, lse_part, BH, Nq, Nk, n_splits,
                                  split_tiles, scale, stream, drop, mask);
    case FA_DTYPE_F16:
        return launch_fwd<_Float16>(L, q, k, v, o, lse, o_part, lse_part, BH, Nq, Nk, n_splits,
                                    split_tiles, scale, stream, drop, mask);
    default:
        return launch_fwd<float>(L, q, k, v, o, lse, o_part, lse_part, BH, Nq, Nk, n_splits,
                                 split_tiles, scale, stream, nullptr, mask);
    }
}

hipError_t launch_merge(fa_dtype_t dtype, int64_t d, const float* o_part, const float* lse_part,
                        int n_parts, int64_t rows, void* o, float* lse, hipStream_t stream)
{
    const int rpb = 256 / (int)(d / 4);
    const int64_t grid = (rows + rpb - 1) / rpb;
    int np = n_parts;
    void* args[] = {(void*)&o_part, (void*)&lse_part, (void*)&np, (void*)&rows, (void*)&o,
                    (void*)&lse};
    return hipLaunchKernel(merge_fn(dtype, d), dim3((unsigned)grid), dim3(256), args, 0, stream);
}

// The key ranges fa_fwd_split uses for a requested count: ranges of whole 64-key
// tiles, as equal as possible, none empty.  Returns the number of ranges and the
// tiles per range.
int split_plan(int64_t Nk, int n_splits, int* tiles_per_split)
{
    const int64_t nkt = (Nk + kKeyTile - 1) / kKeyTile;
    const int64_t s = n_splits < nkt ? n_splits : nkt;
    const int64_t tps = (nkt + s - 1) / s;
    *tiles_per_split = (int)tps;
    return (int)((nkt + tps - 1) / tps);
}

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace

extern "C" fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                              float scale, fa_dtype_t dtype, fa_stream_t stream)
{
    Launch L;
    bool empty;
    const fa_status_t st =
        check_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, false, &L, &empty);
    if (st != FA_OK || empty)
        return st;
    if (d == 64 && dtype != FA_DTYPE_F32 && B * H * ((Nq + L.rows - 1) / L.rows) <= kSmallGridWgs)
        L = dtype == FA_DTYPE_BF16 ? (causal ? mfma16_kg<__bf16, true>() : mfma16_kg<__bf16, false>())
                                   : (causal ? mfma16_kg<_Float16, true>() : mfma16_kg<_Float16, false>());
    const hipError_t err = launch_fwd_any(dtype, L, q, k, v, o, lse, nullptr, nullptr, B * H, Nq,
                                          Nk, 1, 0, scale, reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" fa_status_t fa_fwd_dropout(const void* q, const void* k, const void* v, void* o,
                                      float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                      int64_t d, int causal, float scale, float p_drop,
                                      uint64_t seed, fa_dtype_t dtype, fa_stream_t stream)
{
    const int t = drop_threshold(p_drop);
    if (t < 0)
        return FA_ERR_INVALID_ARG;
    Launch L;
    bool empty;
    const fa_status_t st =
        check_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, false, &L, &empty);
    if (st != FA_OK)
        return st;
    if (dtype == FA_DTYPE_F32)
        return FA_ERR_UNSUPPORTED;
    if (empty)
        return FA_OK;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (t > 0)
        L = dtype == FA_DTYPE_BF16 ? fwd16_drop<__bf16>(d, causal != 0)
                                   : fwd16_drop<_Float16>(d, causal != 0);
    const Dropout drop{(uint32_t)t, seed};
    const hipError_t err = launch_fwd_any(dtype, L, q, k, v, o, lse, nullptr, nullptr, B * H, Nq,
                                          Nk, 1, 0, scale, hs, t > 0 ? &drop : nullptr);
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

namespace {

// Checks of a caller mask [mask_b, mask_h, Nq, ceil(Nk / 32)] words against (B, H, Nq,
// Nk): extents 1 or B / H and a 4-byte aligned pointer (a workgroup's rows of it stay
// below 2^30 bytes: Nk < 2^25 by the forward's limits).  Fills the kernel's view of it.
fa_status_t check_mask(const uint32_t* mask, int64_t mask_b, int64_t mask_h, int64_t B,
                       int64_t H, int64_t Nq, int64_t Nk, MaskArg* out)
{
    if (!mask || !aligned(mask, 4))
        return FA_ERR_INVALID_ARG;
    if ((mask_b != 1 && mask_b != B) || (mask_h != 1 && mask_h != H))
        return FA_ERR_INVALID_ARG;
    const int64_t w = (Nk + 31) / 32;
    out->words = mask;
    out->w = (int)w;
    out->sh = mask_h == 1 ? 0 : Nq * w;
    out->sb = mask_b == 1 ? 0 : mask_h * Nq * w;
    out->H = (int)H;
    return FA_OK;
}

}  // namespace

extern "C" fa_status_t fa_fwd_masked(const void* q, const void* k, const void* v,
                                     const uint32_t* mask, int64_t mask_b, int64_t mask_h,
                                     void* o, float* lse, int64_t B, int64_t H, int64_t Nq,
                                     int64_t Nk, int64_t d, int causal, float scale,
                                     fa_dtype_t dtype, fa_stream_t stream)
{
    Launch L;
    bool empty;
    fa_status_t st =
        check_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, false, &L, &empty);
    if (st != FA_OK || empty)
        return st;
    MaskArg mk;
    st = check_mask(mask, mask_b, mask_h, B, H, Nq, Nk, &mk);
    if (st != FA_OK)
        return st;
    L = fwd_mask_of(dtype, d, causal != 0);
    const hipError_t err = launch_fwd_any(dtype, L, q, k, v, o, lse, nullptr, nullptr, B * H, Nq,
                                          Nk, 1, 0, scale, reinterpret_cast<hipStream_t>(stream),
                                          nullptr, &mk);
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int64_t fa_fwd_split_workspace(int64_t B, int64_t H, int64_t Nq, int64_t d,
                                          int n_splits)
{
    if (B < 0 || H < 0 || Nq < 0 || (d != 64 && d != 128) || n_splits < 1 ||
        n_splits > kMaxSplits)
        return -1;
    const int64_t parts = mul_sat(mul_sat(mul_sat(B, H), Nq), n_splits);
    const int64_t o_bytes = mul_sat(parts, d * 4);
    if (o_bytes > INT64_MAX / 2)
        return -1;  // no buffer of that size exists
    return round_up(o_bytes, kAlign) + parts * 4;
}

namespace {

// The body of fa_fwd_split once the arguments are valid: the unsplit kernel when one
// key range results, else the split kernels into the partials at `workspace` (which
// must hold fa_fwd_split_workspace(...) bytes) and the merge.
fa_status_t split_launch(fa_dtype_t dtype, const Launch& L, const void* q, const void* k,
                         const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t Nq,
                         int64_t Nk, int64_t d, int causal, float scale, int n_splits, int s_eff,
                         int tps, void* workspace, hipStream_t hs)
{
    if (s_eff == 1) {  // one range: the unsplit kernel writes o and lse directly
        Launch L1;
        pick(dtype, d, causal, false, &L1);
        const hipError_t err = launch_fwd_any(dtype, L1, q, k, v, o, lse, nullptr, nullptr, B * H,
                                              Nq, Nk, 1, 0, scale, hs);
        return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
    }
    const int64_t rows = B * H * Nq;
    float* o_part = static_cast<float*>(workspace);
    float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                               round_up((int64_t)n_splits * rows * d * 4, kAlign));
    hipError_t err = launch_fwd_any(dtype, L, q, k, v, nullptr, nullptr, o_part, lse_part, B * H,
                                    Nq, Nk, s_eff, tps, scale, hs);
    if (err != hipSuccess)
        return FA_ERR_LAUNCH;
    err = launch_merge(dtype, d, o_part, lse_part, s_eff, rows, o, lse, hs);
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Grid limits of the split kernels and the merge for s_eff ranges.
bool split_fits(const Launch& L, int64_t B, int64_t H, int64_t Nq, int s_eff)
{
    const int64_t rows = B * H * Nq;
    return (int64_t)s_eff * ((Nq + L.rows - 1) / L.rows) * B * H <= INT32_MAX &&
           (rows + 7) / 8 <= INT32_MAX;
}

}  // namespace

extern "C" fa_status_t fa_fwd_split(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                    int64_t d, int causal, float scale, fa_dtype_t dtype,
                                    int n_splits, void* workspace, int64_t workspace_bytes,
                                    fa_stream_t stream)
{
    if (n_splits < 1 || n_splits > kMaxSplits)
        return FA_ERR_INVALID_ARG;
    Launch L;
    bool empty;
    const fa_status_t st =
        check_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, true, &L, &empty);
    if (st != FA_OK || empty)
        return st;
    int tps;
    const int s_eff = split_plan(Nk, n_splits, &tps);
    if (s_eff > 1) {
        const int64_t need = fa_fwd_split_workspace(B, H, Nq, d, n_splits);
        if (need < 0 || !workspace || !aligned(workspace, 16) || workspace_bytes < need)
            return FA_ERR_INVALID_ARG;
        if (!split_fits(L, B, H, Nq, s_eff))
            return FA_ERR_INVALID_ARG;
    }
    return split_launch(dtype, L, q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, n_splits,
                        s_eff, tps, workspace, reinterpret_cast<hipStream_t>(stream));
}

// ---- fa_fwd_split_static: the partials in a static device array ------------

// The scratch of fa_fwd_split_static.  Each GPU holds its own copy of the array, at an
// address only the runtime knows: host code never uses this name as an address (it is
// a host-side stand-in there), only the per-device address looked up below.
static __device__ __align__(256) char scratch[FA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device id

// Device address of the current GPU's copy of `scratch`, looked up on the first call
// with that GPU current and kept for later calls.
hipError_t scratch_address(void** out)
{
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !p)
            return err != hipSuccess ? err : hipErrorInvalidSymbol;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" fa_status_t fa_fwd_split_static(const void* q, const void* k, const void* v, void* o,
                                           float* lse, int64_t B, int64_t H, int64_t Nq,
                                           int64_t Nk, int64_t d, int causal, float scale,
                                           fa_dtype_t dtype, int n_splits, fa_stream_t stream)
{
    if (n_splits < 1 || n_splits > kMaxSplits)
        return FA_ERR_INVALID_ARG;
    Launch L;
    bool empty;
    const fa_status_t st =
        check_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, true, &L, &empty);
    if (st != FA_OK || empty)
        return st;
    int tps;
    const int s_eff = split_plan(Nk, n_splits, &tps);
    void* ws = nullptr;
    if (s_eff > 1) {
        const int64_t need = fa_fwd_split_workspace(B, H, Nq, d, n_splits);
        if (need < 0 || need > FA_STATIC_SCRATCH_BYTES)
            return FA_ERR_SCRATCH;
        if (!split_fits(L, B, H, Nq, s_eff))
            return FA_ERR_INVALID_ARG;
        if (scratch_address(&ws) != hipSuccess)
            return FA_ERR_LAUNCH;
    }
    return split_launch(dtype, L, q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, n_splits,
                        s_eff, tps, ws, reinterpret_cast<hipStream_t>(stream));
}

extern "C" fa_status_t fa_merge(const float* o_parts, const float* lse_parts, int n_parts,
                                int64_t B, int64_t H, int64_t Nq, int64_t d, void* o, float* lse,
                                fa_dtype_t dtype, fa_stream_t stream)
{
    if (B < 0 || H < 0 || Nq < 0 || n_parts < 1)
        return FA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype))
        return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128)
        return FA_ERR_UNSUPPORTED;
    const int64_t rows = mul_sat(mul_sat(B, H), Nq);
    if (rows == 0)
        return FA_OK;
    if (!o_parts || !lse_parts || !o || !lse)
        return FA_ERR_INVALID_ARG;
    if (!aligned(o_parts, 16) || !aligned(lse_parts, 4) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_INVALID_ARG;
    // the grid is 1-D, 8 rows a workgroup; the parts' element offsets are 64-bit
    if (rows > 8 * (int64_t)INT32_MAX || mul_sat(mul_sat(rows, n_parts), d) == INT64_MAX)
        return FA_ERR_INVALID_ARG;
    const hipError_t err = launch_merge(dtype, d, o_parts, lse_parts, n_parts, rows, o, lse,
                                        reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_split_hint(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                             fa_dtype_t dtype)
{
    Launch L;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (causal != 0 && causal != 1) ||
        !pick(dtype, d, causal, false, &L))
        return 0;
    const int64_t cus = 256;
    const int64_t slots = cus * wgs_per_cu(dtype, d);
    const int64_t wgs = mul_sat(mul_sat(B, H), Nq / L.rows + (Nq % L.rows != 0));
    if (wgs >= slots)
        return 1;
    // each range must keep enough key tiles to amortise its partial-state write and
    // the merge launch: 8 for the 16-bit kernels, 2 for the slower fp32 one
    const int64_t nkt = Nk / kKeyTile + (Nk % kKeyTile != 0);
    const int64_t min_tiles = dtype == FA_DTYPE_F32 ? 2 : 8;
    int64_t s = (slots + wgs - 1) / wgs;
    const int64_t most = nkt / min_tiles > 1 ? nkt / min_tiles : 1;
    if (s > most)
        s = most;
    if (s > 16)
        s = 16;
    return (int)s;
}

// ---- backward ------------------------------------------------------------

namespace {

template <typename T, int D, bool C, bool DR, bool MK>
hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        int64_t BH, int64_t Nq, int64_t Nk, float scale, float* delta,
                        hipStream_t stream, const Dropout& drop, const MaskArg* mask)
{
    fa::BwdParams<T> prm;
    prm.mask = mask ? mask->words : nullptr;
    prm.mask_sb = mask ? mask->sb : 0;
    prm.mask_sh = mask ? mask->sh : 0;
    prm.mask_w = mask ? mask->w : 0;
    prm.H = mask ? mask->H : 1;
    prm.q = static_cast<const T*>(q);
    prm.k = static_cast<const T*>(k);
    prm.v = static_cast<const T*>(v);
    prm.o = static_cast<const T*>(o);
    prm.dout = static_cast<const T*>(dout);
    prm.lse = lse;
    prm.delta = delta;
    prm.dq = static_cast<T*>(dq);
    prm.dk = static_cast<T*>(dk);
    prm.dv = static_cast<T*>(dv);
    prm.Nq = (int)Nq;
    prm.Nk = (int)Nk;
    prm.c2 = scale_log2e(scale);
    prm.scale = scale;
    prm.drop.key0 = (uint32_t)drop.seed;
    prm.drop.key1 = (uint32_t)(drop.seed >> 32);
    prm.drop.t = drop.t;
    prm.drop.keep_scale = (float)(256.0 / (256.0 - (double)drop.t));
    hipError_t err;
    const int64_t rows = BH * Nq;
    if (rows > 0) {  // D = rowsum(dO o O)
        const int rpb = 256 / (D / 4);
        const T* po = prm.o;
        const T* pd = prm.dout;
        int64_t r = rows;
        void* a0[] = {(void*)&po, (void*)&pd, (void*)&delta, (void*)&r};
        err = hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_bwd_delta_kernel<T, D>),
                              dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), a0, 0, stream);
        if (err != hipSuccess)
            return err;
    }
    void* args[] = {(void*)&prm};
    using PK = fa::DkvTile<D>;
    prm.n_tiles = (int)((Nk + PK::KEYS - 1) / PK::KEYS);  // dK, dV (zeros when Nq == 0)
    err = hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_bwd_dkv_kernel<T, D, C, DR, MK>),
                          dim3((unsigned)(prm.n_tiles * BH)), dim3(PK::NT), args, 0, stream);
    if (err != hipSuccess || rows == 0)
        return err;
    using PQ = fa::DqTile<D>;
    prm.n_tiles = (int)((Nq + PQ::ROWS - 1) / PQ::ROWS);  // dQ
    return hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_bwd_dq_kernel<T, D, C, DR, MK>),
                           dim3((unsigned)(prm.n_tiles * BH)), dim3(PQ::NT), args, 0, stream);
}

template <typename T, bool DR, bool MK>
hipError_t launch_bwd_dr(int64_t d, int causal, const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* dout, void* dq, void* dk,
                         void* dv, int64_t BH, int64_t Nq, int64_t Nk, float scale, float* delta,
                         hipStream_t s, const Dropout& dr, const MaskArg* mk)
{
    if (d == 128)
        return causal ? launch_bwd_t<T, 128, true, DR, MK>(q, k, v, o, lse, dout, dq, dk, dv, BH, Nq, Nk, scale, delta, s, dr, mk)
                      : launch_bwd_t<T, 128, false, DR, MK>(q, k, v, o, lse, dout, dq, dk, dv, BH, Nq, Nk, scale, delta, s, dr, mk);
    return causal ? launch_bwd_t<T, 64, true, DR, MK>(q, k, v, o, lse, dout, dq, dk, dv, BH, Nq, Nk, scale, delta, s, dr, mk)
                  : launch_bwd_t<T, 64, false, DR, MK>(q, k, v, o, lse, dout, dq, dk, dv, BH, Nq, Nk, scale, delta, s, dr, mk);
}

// dropout and a caller mask are not combined (fa_bwd_dropout has no mask argument)
template <typename T>
hipError_t launch_bwd_d(int64_t d, int causal, const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dout, void* dq, void* dk,
                        void* dv, int64_t BH, int64_t Nq, int64_t Nk, float scale, float* delta,
                        hipStream_t s, const Dropout& dr, const MaskArg* mk)
{
    if (mk)
        return launch_bwd_dr<T, false, true>(d, causal, q, k, v, o, lse, dout, dq, dk, dv, BH, Nq,
                                             Nk, scale, delta, s, dr, mk);
    return dr.t > 0 ? launch_bwd_dr<T, true, false>(d, causal, q, k, v, o, lse, dout, dq, dk, dv,
                                                    BH, Nq, Nk, scale, delta, s, dr, nullptr)
                    : launch_bwd_dr<T, false, false>(d, causal, q, k, v, o, lse, dout, dq, dk, dv,
                                                     BH, Nq, Nk, scale, delta, s, dr, nullptr);
}

}  // namespace

extern "C" int64_t fa_bwd_workspace(int64_t B, int64_t H, int64_t Nq, int64_t d)
{
    if (B < 0 || H < 0 || Nq < 0 || (d != 64 && d != 128))
        return -1;
    const int64_t bytes = mul_sat(mul_sat(mul_sat(B, H), Nq), 4);
    return bytes > INT64_MAX / 2 ? -1 : round_up(bytes, kAlign);
}

namespace {

fa_status_t bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                     int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                     fa_dtype_t dtype, void* workspace, int64_t workspace_bytes,
                     fa_stream_t stream, const Dropout& drop, const uint32_t* mask = nullptr,
                     int64_t mask_b = 0, int64_t mask_h = 0, bool masked = false)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
        return FA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype))
        return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1)
        return FA_ERR_INVALID_ARG;
    if (!(scale > 0.0f) || !isfinite(scale))
        return FA_ERR_INVALID_ARG;
    if ((d != 64 && d != 128) || dtype == FA_DTYPE_F32)
        return FA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || (Nq == 0 && Nk == 0))
        return FA_OK;  // nothing to compute
    if (Nk == 0)
        return FA_ERR_INVALID_ARG;  // queries without keys: the forward is undefined
    // size limits: in-head offsets are 32-bit, the grids are 1-D (128-row tiles; the
    // delta pass takes 8 rows a workgroup)
    const int64_t lim = INT32_MAX;
    if (mul_sat(Nq, d) > lim || mul_sat(Nk, d) > lim || mul_sat(B, H) > lim)
        return FA_ERR_INVALID_ARG;
    if (B * H * ((Nq + 127) / 128) > lim || B * H * ((Nk + 127) / 128) > lim ||
        B * H * Nq / 8 > lim)
        return FA_ERR_INVALID_ARG;
    if (!k || !v || !dk || !dv || !aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) ||
        !aligned(dv, 16))
        return FA_ERR_INVALID_ARG;
    if (Nq > 0) {
        if (!q || !o || !lse || !dout || !dq || !aligned(q, 16) || !aligned(o, 16) ||
            !aligned(dout, 16) || !aligned(dq, 16) || !aligned(lse, 4))
            return FA_ERR_INVALID_ARG;
        if (!workspace || !aligned(workspace, 16) ||
            workspace_bytes < fa_bwd_workspace(B, H, Nq, d))
            return FA_ERR_INVALID_ARG;
    }
    MaskArg mk;
    if (masked && Nq > 0) {
        const fa_status_t st = check_mask(mask, mask_b, mask_h, B, H, Nq, Nk, &mk);
        if (st != FA_OK)
            return st;
    }
    const MaskArg* mkp = (masked && Nq > 0) ? &mk : nullptr;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    float* delta = static_cast<float*>(workspace);
    const hipError_t err =
        dtype == FA_DTYPE_BF16
            ? launch_bwd_d<__bf16>(d, causal, q, k, v, o, lse, dout, dq, dk, dv, B * H, Nq, Nk,
                                   scale, delta, hs, drop, mkp)
            : launch_bwd_d<_Float16>(d, causal, q, k, v, o, lse, dout, dq, dk, dv, B * H, Nq, Nk,
                                     scale, delta, hs, drop, mkp);
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                              float scale, fa_dtype_t dtype, void* workspace,
                              int64_t workspace_bytes, fa_stream_t stream)
{
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, causal, scale, dtype,
                    workspace, workspace_bytes, stream, Dropout{0u, 0u});
}

extern "C" fa_status_t fa_bwd_masked(const void* q, const void* k, const void* v,
                                     const uint32_t* mask, int64_t mask_b, int64_t mask_h,
                                     const void* o, const float* lse, const void* dout, void* dq,
                                     void* dk, void* dv, int64_t B, int64_t H, int64_t Nq,
                                     int64_t Nk, int64_t d, int causal, float scale,
                                     fa_dtype_t dtype, void* workspace, int64_t workspace_bytes,
                                     fa_stream_t stream)
{
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, causal, scale, dtype,
                    workspace, workspace_bytes, stream, Dropout{0u, 0u}, mask, mask_b, mask_h,
                    true);
}

extern "C" fa_status_t fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                                      const float* lse, const void* dout, void* dq, void* dk,
                                      void* dv, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                      int64_t d, int causal, float scale, float p_drop,
                                      uint64_t seed, fa_dtype_t dtype, void* workspace,
                                      int64_t workspace_bytes, fa_stream_t stream)
{
    const int t = drop_threshold(p_drop);
    if (t < 0)
        return FA_ERR_INVALID_ARG;
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, causal, scale, dtype,
                    workspace, workspace_bytes, stream, Dropout{(uint32_t)t, seed});
}

extern "C" const char* fa_status_str(fa_status_t status)
{
    switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH";
    }
    return "FA_ERR_UNKNOWN";
}

extern "C" int fa_tile_rows(fa_dtype_t dtype, int64_t d, int causal)
{
    if (causal != 0 && causal != 1)
        return 0;
    Launch L;
    return pick(dtype, d, causal, false, &L) ? L.rows : 0;
}
