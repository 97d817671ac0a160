// fa_abi.hip — the C-ABI of libfa.so: argument validation and kernel dispatch.
//
// Declared in include/fa.h.  Every argument error is returned before any HIP call;
// the kernel is enqueued with hipLaunchKernel so that its own launch status is
// returned (no sticky error from earlier, unrelated calls is consumed).
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/fa.h"
#include "fa_fwd_f32.hpp"
#include "fa_fwd_mfma16.hpp"

namespace {

struct Launch {
    const void* fn;  // device function address
    int rows;        // query rows per workgroup
    int threads;     // threads per workgroup
};

template <typename T, int D, bool C>
Launch mfma16()
{
    return Launch{reinterpret_cast<const void*>(&fa::fa_fwd_mfma16_kernel<T, D, C>),
                  fa::Tile16<D>::BR, fa::Tile16<D>::NT};
}

template <int D, bool C>
Launch f32()
{
    return Launch{reinterpret_cast<const void*>(&fa::fa_fwd_f32_kernel<D, C>), fa::TileF32<D>::BR,
                  fa::TileF32<D>::NT};
}

bool pick(fa_dtype_t dtype, int64_t d, int causal, Launch* out)
{
    const bool c = causal != 0;
    if (d != 64 && d != 128)
        return false;
    const bool d128 = d == 128;
    switch (dtype) {
    case FA_DTYPE_BF16:
        *out = d128 ? (c ? mfma16<__bf16, 128, true>() : mfma16<__bf16, 128, false>())
                    : (c ? mfma16<__bf16, 64, true>() : mfma16<__bf16, 64, false>());
        return true;
    case FA_DTYPE_F16:
        *out = d128 ? (c ? mfma16<_Float16, 128, true>() : mfma16<_Float16, 128, false>())
                    : (c ? mfma16<_Float16, 64, true>() : mfma16<_Float16, 64, false>());
        return true;
    case FA_DTYPE_F32:
        *out = d128 ? (c ? f32<128, true>() : f32<128, false>())
                    : (c ? f32<64, true>() : f32<64, false>());
        return true;
    }
    return false;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                              float scale, fa_dtype_t dtype, fa_stream_t stream)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
        return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1)
        return FA_ERR_INVALID_ARG;
    if (!(scale > 0.0f) || !isfinite(scale))
        return FA_ERR_INVALID_ARG;
    Launch L;
    if (!pick(dtype, d, causal, &L))
        return FA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || Nq == 0)
        return FA_OK;  // nothing to compute: no buffer is touched, pointers may be null
    if (!q || !k || !v || !o || !lse)
        return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(lse, 4))
        return FA_ERR_INVALID_ARG;
    if (Nk == 0)
        return FA_ERR_INVALID_ARG;  // softmax over an empty key set is undefined

    // size limits: in-head offsets are 32-bit, the grid is 1-D
    const int64_t lim = INT32_MAX;
    if (Nq * d > lim || Nk * d > lim || B > lim || H > lim || B * H > lim)
        return FA_ERR_INVALID_ARG;
    const int64_t n_qtiles = (Nq + L.rows - 1) / L.rows;
    if (n_qtiles * B * H > lim)
        return FA_ERR_INVALID_ARG;

    // exp(x) = 2^(x * log2 e): fold log2(e) into the scale once, in double
    const float c2 = (float)((double)scale * 1.4426950408889634074);
    int nq = (int)Nq, nk = (int)Nk, nt = (int)n_qtiles;
    void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&lse,
                    (void*)&nq, (void*)&nk, (void*)&nt, (void*)&c2};
    const hipError_t err = hipLaunchKernel(L.fn, dim3((unsigned)(n_qtiles * B * H)),
                                           dim3((unsigned)L.threads), args, 0,
                                           reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" const char* fa_status_str(fa_status_t status)
{
    switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH";
    }
    return "FA_ERR_UNKNOWN";
}

extern "C" int fa_tile_rows(fa_dtype_t dtype, int64_t d, int causal)
{
    if (causal != 0 && causal != 1)
        return 0;
    Launch L;
    return pick(dtype, d, causal, &L) ? L.rows : 0;
}
