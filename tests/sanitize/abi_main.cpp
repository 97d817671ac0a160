// Sanitizer driver for the host side of the C-ABI (csrc/fa_abi.hip): every entry point
// with arguments that its checks refuse before any HIP call (null, misaligned and
// out-of-range arguments, sizes past the 32-bit limits, bad masks and workspaces),
// plus the size and hint queries.  Built host-only with -fsanitize=address,undefined;
// any finding aborts the run.  Prints "ok" on success.
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/fa.h"

int main()
{
    const uintptr_t P = 0x10000;  // an aligned, non-null address the checks never follow
    void* p = reinterpret_cast<void*>(P);
    float* pf = reinterpret_cast<float*>(P);
    const uint32_t* pm = reinterpret_cast<const uint32_t*>(P);
    int bad = 0, n = 0;
    auto expect = [&](fa_status_t got, fa_status_t want) {
        ++n;
        if (got != want) {
            std::printf("case %d: got %d want %d\n", n, (int)got, (int)want);
            ++bad;
        }
    };
    const fa_dtype_t bf = FA_DTYPE_BF16;
    expect(fa_fwd(nullptr, p, p, p, pf, 1, 1, 8, 8, 64, 0, 0.125f, bf, nullptr), FA_ERR_INVALID_ARG);
    expect(fa_fwd(p, p, p, p, pf, 1, 1, 8, 8, 96, 0, 0.125f, bf, nullptr), FA_ERR_UNSUPPORTED);
    expect(fa_fwd(p, p, p, p, pf, -1, 1, 8, 8, 64, 0, 0.125f, bf, nullptr), FA_ERR_INVALID_ARG);
    expect(fa_fwd(p, p, p, p, pf, 1, 1, 8, 0, 64, 0, 0.125f, bf, nullptr), FA_ERR_INVALID_ARG);
    expect(fa_fwd(p, p, p, p, pf, 1, 1, INT64_C(1) << 40, 8, 64, 0, 0.125f, bf, nullptr),
           FA_ERR_INVALID_ARG);
    expect(fa_fwd(p, p, p, p, pf, INT64_C(1) << 40, INT64_C(1) << 40, 8, 8, 64, 0, 0.125f, bf,
                  nullptr), FA_ERR_INVALID_ARG);
    expect(fa_fwd(p, p, p, p, pf, 1, 1, INT64_C(1) << 60, 8, 128, 0, 0.125f, bf, nullptr),
           FA_ERR_INVALID_ARG);
    expect(fa_fwd_masked(p, p, p, pm, 1, 1, p, pf, 1, 1, 8, INT64_C(1) << 60, 64, 0, 0.125f, bf,
                         nullptr), FA_ERR_INVALID_ARG);
    expect(fa_bwd(p, p, p, p, pf, p, p, p, p, INT64_C(1) << 40, INT64_C(1) << 40, 64, 64, 128, 0,
                  0.125f, bf, p, INT64_MAX, nullptr), FA_ERR_INVALID_ARG);
    expect(fa_bwd(p, p, p, p, pf, p, p, p, p, 1, 1, INT64_C(1) << 60, 64, 128, 0, 0.125f, bf, p,
                  INT64_MAX, nullptr), FA_ERR_INVALID_ARG);
    expect(fa_merge(pf, pf, 2, INT64_C(1) << 40, INT64_C(1) << 40, 8, 64, p, pf, bf, nullptr),
           FA_ERR_INVALID_ARG);
    expect(fa_merge(pf, pf, INT32_MAX, 1 << 20, 1 << 10, 1 << 3, 128, p, pf, bf, nullptr),
           FA_ERR_INVALID_ARG);
    expect(fa_fwd_split(p, p, p, p, pf, INT64_C(1) << 40, INT64_C(1) << 40, 64, 640, 128, 0,
                        0.125f, bf, 4, p, INT64_MAX, nullptr), FA_ERR_INVALID_ARG);
    expect(fa_fwd(p, p, p, p, pf, 1, 1, 8, 8, 64, 0, -1.0f, bf, nullptr), FA_ERR_INVALID_ARG);
    expect(fa_fwd(p, p, p, p, pf, 0, 1, 8, 8, 64, 0, 0.125f, bf, nullptr), FA_OK);
    expect(fa_fwd_masked(p, p, p, nullptr, 1, 1, p, pf, 1, 2, 8, 8, 64, 0, 0.125f, bf, nullptr),
           FA_ERR_INVALID_ARG);
    expect(fa_fwd_masked(p, p, p, pm, 3, 1, p, pf, 2, 2, 8, 8, 64, 0, 0.125f, bf, nullptr),
           FA_ERR_INVALID_ARG);
    expect(fa_fwd_split(p, p, p, p, pf, 1, 2, 64, 640, 128, 0, 0.125f, bf, 4, p, 16, nullptr),
           FA_ERR_INVALID_ARG);
    expect(fa_fwd_split(p, p, p, p, pf, 1, 2, 64, 640, 128, 0, 0.125f, bf, 0, p, 1 << 20, nullptr),
           FA_ERR_INVALID_ARG);
    expect(fa_fwd_split_static(p, p, p, p, pf, 64, 16, 4096, 128, 128, 0, 0.125f, bf, 2, nullptr),
           FA_ERR_SCRATCH);
    expect(fa_merge(pf, pf, 0, 1, 1, 8, 64, p, pf, bf, nullptr), FA_ERR_INVALID_ARG);
    expect(fa_merge(pf, pf, 2, 1, 1, 8, 80, p, pf, bf, nullptr), FA_ERR_UNSUPPORTED);
    expect(fa_bwd(p, p, p, p, pf, p, p, p, p, 1, 2, 64, 64, 128, 0, 0.125f, FA_DTYPE_F32, p, 1 << 20,
                  nullptr), FA_ERR_UNSUPPORTED);
    expect(fa_bwd(p, p, p, p, pf, p, p, p, p, 1, 2, 64, 64, 128, 0, 0.125f, bf, p, 4, nullptr),
           FA_ERR_INVALID_ARG);
    expect(fa_bwd_masked(p, p, p, nullptr, 1, 1, p, pf, p, p, p, p, 1, 2, 64, 64, 128, 0, 0.125f, bf,
                         p, 1 << 20, nullptr), FA_ERR_INVALID_ARG);
    expect(fa_fwd_dropout(p, p, p, p, pf, 1, 2, 64, 64, 128, 0, 0.125f, 1.5f, 7, bf, nullptr),
           FA_ERR_INVALID_ARG);
    expect(fa_bwd_dropout(p, p, p, p, pf, p, p, p, p, 1, 2, 64, 64, 128, 0, 0.125f, -0.1f, 7, bf, p,
                          1 << 20, nullptr), FA_ERR_INVALID_ARG);
    // unknown enum values, as a C caller may pass them
    const fa_dtype_t odd = static_cast<fa_dtype_t>(99);
    expect(fa_fwd(p, p, p, p, pf, 1, 1, 8, 8, 64, 0, 0.125f, odd, nullptr), FA_ERR_INVALID_ARG);
    expect(fa_fwd_split(p, p, p, p, pf, 1, 2, 64, 640, 128, 0, 0.125f, odd, 2, p, 1 << 30, nullptr),
           FA_ERR_INVALID_ARG);
    expect(fa_merge(pf, pf, 2, 1, 1, 8, 64, p, pf, odd, nullptr), FA_ERR_INVALID_ARG);
    expect(fa_bwd(p, p, p, p, pf, p, p, p, p, 1, 2, 64, 64, 128, 0, 0.125f, odd, p, 1 << 20,
                  nullptr), FA_ERR_INVALID_ARG);
    // size queries past int64: refused, not wrapped
    const int64_t huge = INT64_C(1) << 40;
    ++n;
    if (fa_fwd_split_workspace(huge, huge, huge, 128, 16) != -1 ||
        fa_bwd_workspace(huge, huge, huge, 128) != -1 ||
        fa_split_hint(huge, huge, huge, huge, 128, 1, bf) != 1) {
        std::printf("case %d: huge size queries\n", n);
        ++bad;
    }
    ++n;
    if (fa_fwd_split_workspace(-1, 1, 1, 64, 2) != -1 || fa_bwd_workspace(1, 1, 1, 96) != -1 ||
        fa_split_hint(1, 1, 256, 16384, 128, 0, bf) < 1 || fa_split_hint(1, 1, 256, 16384, 128, 0,
                                                                         odd) != 0 ||
        fa_tile_rows(bf, 128, 1) <= 0 || fa_tile_rows(odd, 128, 1) != 0 ||
        std::string(fa_status_str(static_cast<fa_status_t>(99))) != "FA_ERR_UNKNOWN" ||
        std::string(fa_status_str(FA_ERR_SCRATCH)) != "FA_ERR_SCRATCH") {
        std::printf("case %d: size queries\n", n);
        ++bad;
    }
    if (bad) {
        std::printf("%d of %d cases failed\n", bad, n);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
