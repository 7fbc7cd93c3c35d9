// Drives the host side of the C ABI (include/w4a4.h) in a build with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code: the
// layout helpers, the permutation, the workspace and kernel-name queries,
// empty calls, and argument checks that must reject a call before any device
// work (no kernel is launched; no GPU is needed). Exit status 0 when every
// call returned what the header states.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "w4a4.h"

static int failures = 0;
#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);  \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

// A 256-byte aligned, never dereferenced address (every call below fails or
// returns before touching its buffers).
static void *fake(uintptr_t off = 0) { return reinterpret_cast<void *>(uintptr_t(1) << 20 | off); }

int main() {
    CHECK(std::strcmp(w4a4_status_string(W4A4_OK), "W4A4_OK") == 0);
    CHECK(std::strcmp(w4a4_status_string(99), "W4A4_ERR_UNKNOWN") == 0);
    for (int32_t K_n : {0, 1, 127, 128, 129, 21760})
        CHECK(w4a4_pitch4_bytes(K_n) == (int64_t)((K_n + 127) / 128) * 64);
    for (int32_t n : {0, 1, 64, 65, 256})
        CHECK(w4a4_pitch8_bytes(n) == (int64_t)((n + 63) / 64) * 64);
    CHECK(w4a4_num_groups(3968, 128) == 31 && w4a4_num_groups(240, 0) == 1 && w4a4_num_groups(0, 0) == 0);
    CHECK(w4a4_num_groups(100, 128) < 0);

    // permutation: definition and rejects
    std::vector<int32_t> perm(4096), outl = {7, 300, 4095};
    CHECK(w4a4_make_perm(4096, outl.data(), 3, perm.data()) == W4A4_OK);
    CHECK(perm[4093] == 7 && perm[4094] == 300 && perm[4095] == 4095 && perm[7] == 8);
    int32_t rep[2] = {1, 1}, out[1] = {9};
    CHECK(w4a4_make_perm(9, rep, 2, perm.data()) == W4A4_ERR_INVALID_ARG);
    CHECK(w4a4_make_perm(9, out, 1, perm.data()) == W4A4_ERR_INVALID_ARG);

    // queries
    for (int32_t M : {1, 8, 128, 256, 2048})
        CHECK(w4a4_outlier_gemm_kernel_name(M, 8192, 8192, 128, 128) != nullptr);
    CHECK(w4a4_outlier_gemm_fp6_kernel_name(2048, 4096, 4096, 128, 128) != nullptr);
    CHECK(w4a4_quant_gemm_workspace_bytes(256, 8192, 8192, 128, 128) > 0);
    CHECK(w4a4_quant_gemm_fp6_workspace_bytes(8192, 8192, 22016, 256, 0) > 0);
    CHECK(w4a4_select_outliers_workspace_bytes(4096, 4096) > 0);
    CHECK(w4a4_u6_bytes(37, 640) > 0 && w4a4_u6_bytes(0, 640) == 0);
    CHECK(w4a4_quant_gemm_static_max_bytes() > 0);

    // empty calls succeed without touching pointers
    CHECK(w4a4_quant_reorder_act(nullptr, 256, nullptr, 0, 256, 16, 0, nullptr, nullptr, nullptr, nullptr,
                                 nullptr) == W4A4_OK);
    CHECK(w4a4_quant_reorder_act_u6(nullptr, 256, nullptr, 0, 256, 16, 0, nullptr, nullptr, nullptr, nullptr,
                                    nullptr) == W4A4_OK);

    // argument checks that reject before any device work
    CHECK(w4a4_quant_reorder_act(fake(), 256, (int32_t *)fake(), 4, 0, 16, 0, fake(), fake(), (float *)fake(),
                                 (float *)fake(), nullptr) == W4A4_ERR_INVALID_ARG);
    CHECK(w4a4_quant_reorder_act(fake(), 100, (int32_t *)fake(), 4, 256, 16, 0, fake(), fake(), (float *)fake(),
                                 (float *)fake(), nullptr) == W4A4_ERR_INVALID_ARG);
    CHECK(w4a4_quant_reorder_act(fake(2), 256, (int32_t *)fake(), 4, 256, 16, 0, fake(), fake(),
                                 (float *)fake(), (float *)fake(), nullptr) == W4A4_ERR_ALIGNMENT);
    CHECK(w4a4_quant_reorder_act(fake(), 256, (int32_t *)fake(), 4, 256, 16, 100, fake(), fake(),
                                 (float *)fake(), (float *)fake(), nullptr) == W4A4_ERR_INVALID_ARG);
    CHECK(w4a4_quant_reorder_act(fake(), 24584, (int32_t *)fake(), 4, 24584, 0, 0, fake(), fake(),
                                 (float *)fake(), (float *)fake(), nullptr) == W4A4_ERR_UNSUPPORTED);
    CHECK(w4a4_quant_reorder_act_u6(fake(), 272, (int32_t *)fake(), 4, 272, 16, 64, fake(), fake(),
                                    (float *)fake(), (float *)fake(), nullptr) == W4A4_ERR_UNSUPPORTED);
    CHECK(w4a4_quant_reorder_act_u6(fake(), 256, (int32_t *)fake(), 4, 256, 16, 0, fake(8), fake(),
                                    (float *)fake(), (float *)fake(), nullptr) == W4A4_ERR_ALIGNMENT);
    CHECK(w4a4_rmsnorm_quant_reorder_act(fake(), 256, nullptr, 1e-6f, (int32_t *)fake(), 4, 256, 16, 0, fake(),
                                         fake(), (float *)fake(), (float *)fake(), nullptr,
                                         nullptr) == W4A4_ERR_INVALID_ARG);
    const float *fs = (const float *)fake();
    CHECK(w4a4_outlier_gemm(fake(), fake(), fs, fs, fake(), fake(), fs, fs, 4, 8, 0, 16, 0, fake(), 8, nullptr, 0,
                            nullptr) == W4A4_ERR_INVALID_ARG);
    CHECK(w4a4_outlier_gemm(fake(), fake(), fs, fs, fake(), fake(), fs, fs, 4, 8, 256, 16, 0, fake(), 4, nullptr, 0,
                            nullptr) == W4A4_ERR_INVALID_ARG);
    CHECK(w4a4_outlier_gemm_fp6(fake(), fake(), fs, fs, fake(), fake(), fs, fs, 4, 8, 4352, 256, 256, fake(), 8,
                                nullptr) == W4A4_ERR_UNSUPPORTED);
    CHECK(w4a4_w4a8_gemm(fake(), fs, fake(), fs, 4, 8, 100, 0, fake(), 8, nullptr) != W4A4_OK);
    CHECK(w4a4_kv_quant(fake(), 128, 4, 1, 100, 4, nullptr, 4, fake(), (float *)fake(), nullptr) != W4A4_OK);
    CHECK(w4a4_select_outliers(fake(), 4096, 16, 4096, 5000, (int32_t *)fake(), (int32_t *)fake(), nullptr,
                               fake(), 1 << 20, nullptr) == W4A4_ERR_INVALID_ARG);

    if (failures)
        std::fprintf(stderr, "%d checks failed\n", failures);
    else
        std::printf("ABI host sanitizer run: all checks passed\n");
    return failures ? 1 : 0;
}
