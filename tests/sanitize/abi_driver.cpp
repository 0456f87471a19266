// abi_driver.cpp -- the host side of liblora_mi355x (include/lora.h) under AddressSanitizer
// and UndefinedBehaviorSanitizer: every entry point called with arguments its validation
// rejects (and M = 0 no-ops), the sizing functions over many shapes, every status string.
// No call here reaches a kernel launch, so no GPU is needed; fake device addresses are never
// dereferenced.  Built by tests/test_sanitizers.py with the library's sources; exit status 0
// when every call returned the status expected of it.  Test infrastructure.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lora.h"

static int failures = 0;
#define EXPECT(call, want)                                                                  \
    do {                                                                                    \
        int got_ = (int)(call);                                                             \
        if (got_ != (int)(want)) {                                                          \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
                    got_, (int)(want));                                                     \
            ++failures;                                                                     \
        }                                                                                   \
    } while (0)

static void *const F = reinterpret_cast<void *>(uintptr_t(1) << 20);  // 256-byte aligned
static float *const FF = static_cast<float *>(F);
static int32_t *const FI = static_cast<int32_t *>(F);
static void *off(size_t b) { return static_cast<char *>(F) + b; }

int main() {
    // sizing
    EXPECT(lora_max_tiles(0, 4), 0);
    EXPECT(lora_max_tiles(16, 4), 5);
    EXPECT(lora_max_tiles(-3, 4), 0);
    const int rs[] = {0, 1, 7, 8, 12, 16, 24, 33, 64, 65};
    const int Ms[] = {0, 1, 64, 128, 129, 256, 257, 767, 768, 1024, 4096};
    const int ds[] = {8, 120, 4096, 4104, 11008};
    for (int r : rs)
        for (int M : Ms)
            for (int d : ds) {
                const size_t b = lora_workspace_bytes(M, d, 4096, r, 32);
                const bool ok = r >= 1 && r <= 64;
                if ((b != 0) != (ok && M > 0) || b % 256 != 0) {
                    fprintf(stderr, "workspace bytes %zu for M %d d %d r %d\n", b, M, d, r);
                    ++failures;
                }
            }
    for (int r : rs)
        for (int M : {0, 1, 64, 2048, 2049})
            for (int E : {0, 1, 32, 4096, 4097}) {
                const size_t b = lora_moe_workspace_bytes(M, 4, E, 2880, 2880, r, 8);
                const bool ok = r >= 8 && r % 8 == 0 && r <= 64 && M > 0 && M <= 2048 && E >= 1 &&
                                E <= 4096;
                if ((b != 0) != ok || b % 256 != 0) {
                    fprintf(stderr, "moe workspace bytes %zu for M %d E %d r %d\n", b, M, E, r);
                    ++failures;
                }
            }
    for (int s = -1; s <= 12; ++s) {
        const char *str = lora_status_string(static_cast<lora_status_t>(s));
        if (!str || !*str) ++failures;
    }
    if (!lora_last_hip_error()) ++failures;

    lora_segments_t seg{FI, FI, FI, FI, FI};
    lora_segments_t bad_seg{FI, nullptr, FI, FI, FI};
    const size_t ws = lora_workspace_bytes(64, 4096, 4096, 16, 32);

    // segments
    EXPECT(lora_build_segments(FI, -1, 8, seg, nullptr), LORA_ERR_SHAPE);
    EXPECT(lora_build_segments(FI, 8, 0, seg, nullptr), LORA_ERR_SHAPE);
    EXPECT(lora_build_segments(nullptr, 8, 4, seg, nullptr), LORA_ERR_NULL);
    EXPECT(lora_build_segments(FI, 8, 4, bad_seg, nullptr), LORA_ERR_NULL);
    EXPECT(lora_build_segments(static_cast<int32_t *>(off(2)), 8, 4, seg, nullptr), LORA_ERR_ALIGN);
    EXPECT(lora_build_segments(FI, 0, 4, seg, nullptr), LORA_OK);

    // shrink / expand (padded and compact)
    EXPECT(lora_shrink(F, F, nullptr, 64, 4096, 65, 32, seg, FF, F, ws, nullptr), LORA_ERR_RANK);
    EXPECT(lora_shrink(F, F, nullptr, 64, 12, 16, 32, seg, FF, F, ws, nullptr), LORA_ERR_SHAPE);
    EXPECT(lora_shrink(nullptr, F, nullptr, 64, 4096, 16, 32, seg, FF, F, ws, nullptr), LORA_ERR_NULL);
    EXPECT(lora_shrink(F, F, nullptr, 64, 4096, 16, 32, seg, FF, F, 16, nullptr), LORA_ERR_WORKSPACE);
    EXPECT(lora_shrink_compact(F, F, FI, nullptr, 64, 64, 4096, 16, 32, seg, FF, F, ws, nullptr),
           LORA_ERR_NULL);
    EXPECT(lora_shrink_compact(F, F, FI, FI, 0, 64, 4096, 16, 32, seg, FF, F, ws, nullptr),
           LORA_ERR_SHAPE);
    EXPECT(lora_expand(FF, F, FF, nullptr, 64, 4096, 16, 32, seg, F, static_cast<lora_dtype_t>(3),
                       nullptr), LORA_ERR_DTYPE);
    EXPECT(lora_expand(FF, F, FF, nullptr, 64, 4100, 16, 32, seg, F, LORA_BF16, nullptr),
           LORA_ERR_SHAPE);
    EXPECT(lora_expand_compact(FF, F, FF, FI, FI, 1 << 20, 64, 4096, 16, 32, seg, F, LORA_BF16,
                               nullptr), LORA_ERR_SHAPE);

    // the layer and its variants
    const lora_mode_t dec = LORA_MODE_DECODE;
    EXPECT(lora_linear(F, F, F, F, FF, nullptr, FI, -1, 4096, 4096, 16, 32, nullptr, F, LORA_BF16,
                       dec, F, ws, nullptr), LORA_ERR_SHAPE);
    EXPECT(lora_linear(F, F, F, F, FF, nullptr, FI, 64, 4096, 4096, 0, 32, nullptr, F, LORA_BF16,
                       dec, F, ws, nullptr), LORA_ERR_RANK);
    EXPECT(lora_linear(F, F, F, F, FF, nullptr, FI, 64, 4096, 4096, 16, 32, nullptr, F, LORA_BF16,
                       static_cast<lora_mode_t>(7), F, ws, nullptr), LORA_ERR_MODE);
    EXPECT(lora_linear(F, F, F, F, FF, nullptr, nullptr, 64, 4096, 4096, 16, 32, nullptr, F,
                       LORA_BF16, dec, F, ws, nullptr), LORA_ERR_NULL);
    EXPECT(lora_linear(off(2), F, F, F, FF, nullptr, FI, 64, 4096, 4096, 16, 32, nullptr, F,
                       LORA_BF16, dec, F, ws, nullptr), LORA_ERR_ALIGN);
    EXPECT(lora_linear(F, F, F, F, FF, nullptr, FI, 64, 4096, 4096, 16, 32, &bad_seg, F, LORA_BF16,
                       dec, F, ws, nullptr), LORA_ERR_NULL);
    EXPECT(lora_linear(F, F, F, F, FF, nullptr, FI, 64, 4096, 4096, 16, 32, nullptr, F, LORA_BF16,
                       dec, F, ws - 1, nullptr), LORA_ERR_WORKSPACE);
    EXPECT(lora_linear(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4096, 4096,
                       16, 32, nullptr, nullptr, LORA_BF16, dec, nullptr, 0, nullptr), LORA_OK);
    EXPECT(lora_linear_compact(F, F, F, F, FF, FI, FI, 0, FI, 64, 4096, 4096, 16, 32, nullptr, F,
                               LORA_BF16, dec, F, ws, nullptr), LORA_ERR_SHAPE);
    EXPECT(lora_linear_compact(F, F, F, F, FF, nullptr, FI, 64, FI, 64, 4096, 4096, 16, 32, nullptr,
                               F, LORA_BF16, dec, F, ws, nullptr), LORA_ERR_NULL);
    EXPECT(lora_linear_noalloc(F, F, F, F, FF, nullptr, FI, 512, 4096, 11008, 16, 32, nullptr, F,
                               LORA_BF16, dec, nullptr), LORA_ERR_WORKSPACE);
    EXPECT(lora_linear_noalloc(F, F, F, F, FF, nullptr, FI, 64, 4096, 4096, 99, 32, nullptr, F,
                               LORA_BF16, dec, nullptr), LORA_ERR_RANK);
    EXPECT(lora_linear_fp8w(F, F, FF, F, F, FF, nullptr, FI, 257, 4096, 4096, 16, 32, nullptr, F,
                            LORA_BF16, dec, F, ws, nullptr), LORA_ERR_SHAPE);
    EXPECT(lora_linear_fp8w(F, F, FF, F, F, FF, nullptr, FI, 64, 4096, 4096, 16, 32, nullptr, F,
                            LORA_BF16, LORA_MODE_PREFILL, F, ws, nullptr), LORA_ERR_MODE);
    EXPECT(lora_linear_fp8w(F, F, nullptr, F, F, FF, nullptr, FI, 64, 4096, 4096, 16, 32, nullptr,
                            F, LORA_BF16, dec, F, ws, nullptr), LORA_ERR_NULL);

    // measurement aids: their own argument checks first, then the call's validation
    float ms[4];
    const char *names[4];
    int32_t nk = 7;
    EXPECT(lora_linear_profiled(F, F, F, F, FF, nullptr, FI, 64, 4096, 4096, 16, 32, nullptr, F,
                                LORA_BF16, dec, F, ws, nullptr, nullptr, names, 4, &nk),
           LORA_ERR_NULL);
    EXPECT(lora_linear_profiled(F, F, F, F, FF, nullptr, FI, 64, 4096, 4096, 16, 32, nullptr, F,
                                LORA_BF16, dec, F, 8, nullptr, ms, names, 4, &nk),
           LORA_ERR_WORKSPACE);
    EXPECT(nk, 0);
    EXPECT(lora_linear_compact_profiled(F, F, F, F, FF, FI, FI, 0, FI, 64, 4096, 4096, 16, 32,
                                        nullptr, F, LORA_BF16, dec, F, ws, nullptr, ms, names, 4,
                                        &nk), LORA_ERR_SHAPE);
    EXPECT(lora_linear_fp8w_profiled(F, F, FF, F, F, FF, nullptr, FI, 64, 4100, 4096, 16, 32,
                                     nullptr, F, LORA_BF16, dec, F, ws, nullptr, ms, names, 4, &nk),
           LORA_ERR_SHAPE);

    // MoE
    const size_t mws = lora_moe_workspace_bytes(64, 4, 32, 2880, 2880, 16, 8);
    EXPECT(lora_moe_linear(F, F, F, F, FF, nullptr, FI, FI, FF, 64, 4, 32, 2880, 2880, 12, 8, F,
                           LORA_BF16, dec, F, mws, nullptr), LORA_ERR_RANK);
    EXPECT(lora_moe_linear(F, F, F, F, FF, nullptr, FI, FI, FF, 2049, 4, 32, 2880, 2880, 16, 8, F,
                           LORA_BF16, dec, F, mws, nullptr), LORA_ERR_SHAPE);
    EXPECT(lora_moe_linear(F, F, F, F, FF, nullptr, FI, nullptr, FF, 64, 4, 32, 2880, 2880, 16, 8,
                           F, LORA_BF16, dec, F, mws, nullptr), LORA_ERR_NULL);
    EXPECT(lora_moe_linear(F, F, F, F, FF, nullptr, FI, FI, static_cast<float *>(off(2)), 64, 4, 32,
                           2880, 2880, 16, 8, F, LORA_BF16, dec, F, mws, nullptr), LORA_ERR_ALIGN);
    EXPECT(lora_moe_linear(F, F, F, F, FF, nullptr, FI, FI, FF, 64, 4, 32, 2880, 2880, 16, 8, F,
                           LORA_BF16, dec, F, mws - 1, nullptr), LORA_ERR_WORKSPACE);
    EXPECT(lora_moe_linear(F, F, F, F, FF, nullptr, FI, FI, FF, 64, 4, 32, 2880, 2880, 16, 8, F,
                           LORA_BF16, LORA_MODE_PREFILL, F, mws, nullptr), LORA_ERR_MODE);
    EXPECT(lora_moe_linear(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, 0, 4, 32, 2880, 2880, 16, 8, nullptr, LORA_BF16, dec, nullptr,
                           0, nullptr), LORA_OK);
    EXPECT(lora_moe_linear_profiled(F, F, F, F, FF, nullptr, FI, FI, FF, 64, 4, 32, 2880, 2880, 16,
                                    8, F, LORA_BF16, dec, F, mws, nullptr, ms, names, -1, &nk),
           LORA_ERR_NULL);

    if (failures) {
        fprintf(stderr, "%d unexpected results\n", failures);
        return 1;
    }
    printf("abi driver: all calls returned the expected status\n");
    return 0;
}
