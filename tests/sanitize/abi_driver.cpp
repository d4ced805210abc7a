// Calls every entry point of libw4a8 (include/w4a8.h) with arguments that
// its host-side validation must reject, and with valid arguments that then
// reach the HIP runtime (on a machine without a GPU the device query fails:
// W4A8_ERR_HIP or W4A8_ERR_UNSUPPORTED).  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of the library, so every
// validation path, the plan and workspace arithmetic and the status
// strings run instrumented.  Fake device pointers are never dereferenced.
// Test infrastructure: only tests/test_sanitizers.py builds and runs it.
#include <cstdio>
#include <cstdint>

#include "w4a8.h"

static int fails = 0;
#define EXPECT(call, want)                                                            \
    do {                                                                              \
        const int got_ = (int)(call);                                                 \
        if (got_ != (int)(want)) {                                                    \
            std::fprintf(stderr, "line %d: %s -> %d, want %d\n", __LINE__, #call, got_, \
                         (int)(want));                                                \
            ++fails;                                                                  \
        }                                                                             \
    } while (0)
#define EXPECT_RUNTIME(call)                                                          \
    do {                                                                              \
        const int got_ = (int)(call);                                                 \
        if (got_ != W4A8_ERR_HIP && got_ != W4A8_ERR_UNSUPPORTED && got_ != W4A8_OK) { \
            std::fprintf(stderr, "line %d: %s -> %d\n", __LINE__, #call, got_);      \
            ++fails;                                                                  \
        }                                                                             \
    } while (0)

int main() {
    auto* A = reinterpret_cast<void*>(uintptr_t(0x10000));
    auto* b = reinterpret_cast<uint8_t*>(A);
    auto* i8 = reinterpret_cast<int8_t*>(A);
    auto* f = reinterpret_cast<float*>(A);
    auto* i32 = reinterpret_cast<int32_t*>(A);
    auto* mis = reinterpret_cast<uint8_t*>(uintptr_t(0x10004));

    for (int s = -1; s < 9; ++s)
        if (!w4a8_status_str((w4a8_status_t)s)) ++fails;
    EXPECT(w4a8_layout_version(), W4A8_LAYOUT_VERSION);
    (void)w4a8_last_hip_error();
    // workspace sizes over a spread of shapes (plan arithmetic, including
    // the largest the extent limits allow)
    size_t total = 0;
    const int Ms[] = {0, 1, 16, 63, 64, 65, 128, 129, 255, 256, 1000, 4096, 65535};
    const int Ns[] = {0, 64, 256, 4096, 8192, 28672, 1 << 20};
    const int Ks[] = {128, 1024, 8192, 28672, 65536};
    for (int m : Ms)
        for (int n : Ns)
            for (int k : Ks)
                for (int sk : {0, 1, 4}) {
                    const size_t w = w4a8_workspace_size(m, n, k, sk);
                    if (w > W4A8_NOALLOC_SCRATCH_BYTES) ++fails;  // every plan fits the static scratch
                    total += w;
                    // the plan query over the same shapes: a valid shape gets a
                    // plan whose split count and K parts fit its K-steps
                    int kern = -1, rows = 0, chans = 0, splits = 0, parts = 0;
                    const w4a8_status_t st =
                        w4a8_gemm_plan(m, n, k, sk, &kern, &rows, &chans, &splits, &parts);
                    if (st == W4A8_OK) {
                        if (kern < 0 || kern > 2 || rows <= 0 || chans <= 0 || splits < 1 ||
                            parts < 1 || splits * parts > k / 128)
                            ++fails;
                        total += (size_t)(kern + rows + chans + splits + parts);
                    } else if (st != W4A8_ERR_SHAPE) {
                        ++fails;
                    }
                }
    EXPECT(w4a8_workspace_size(-5, 256, 128, 0), 0);
    {
        int v[5];
        EXPECT(w4a8_gemm_plan(16, 256, 128, 0, nullptr, v + 1, v + 2, v + 3, v + 4),
               W4A8_ERR_NULL_PTR);
        EXPECT(w4a8_gemm_plan(-1, 256, 128, 0, v, v + 1, v + 2, v + 3, v + 4), W4A8_ERR_SHAPE);
    }

    // pack
    EXPECT(w4a8_pack(nullptr, 64, 256, 64, 127, 0, b, b, b, f, nullptr), W4A8_ERR_NULL_PTR);
    EXPECT(w4a8_pack(f, 64, 200, 64, 127, 0, b, b, b, f, nullptr), W4A8_ERR_SHAPE);
    EXPECT(w4a8_pack(f, 64, 256, 32, 127, 0, b, b, b, f, nullptr), W4A8_ERR_SHAPE);
    EXPECT(w4a8_pack(f, 64, 256, 64, 128, 0, b, b, b, f, nullptr), W4A8_ERR_SHAPE);
    EXPECT(w4a8_pack(f, 64, 256, 64, 127, 9, b, b, b, f, nullptr), W4A8_ERR_UNSUPPORTED);
    EXPECT(w4a8_pack(f, 64, 256, 64, 127, 0, b, mis, b, f, nullptr), W4A8_ERR_ALIGNMENT);
    EXPECT(w4a8_pack(f, 0, 256, 64, 127, 0, nullptr, nullptr, nullptr, nullptr, nullptr), W4A8_OK);
    EXPECT_RUNTIME(w4a8_pack(f, 64, 256, 64, 127, 0, b, b, b, f, nullptr));
    EXPECT_RUNTIME(w4a8_pack(f, 64, 256, 0, 0, 1, b, nullptr, nullptr, f, nullptr));
    // activation quantisers
    for (int it = 0; it < 4; ++it) {
        const int want_bad = it == 3 ? W4A8_ERR_UNSUPPORTED : W4A8_ERR_SHAPE;
        EXPECT(w4a8_quant_act_ex(A, it, 4, 60, i8, f, nullptr), want_bad);
        EXPECT(w4fp8_quant_act_ex(A, it, 4, 60, b, f, nullptr), want_bad);
        if (it < 3) {
            EXPECT(w4a8_quant_act_ex(nullptr, it, 4, 64, i8, f, nullptr), W4A8_ERR_NULL_PTR);
            EXPECT(w4fp8_quant_act_ex(A, it, 4, 64, mis, f, nullptr), W4A8_ERR_ALIGNMENT);
            EXPECT_RUNTIME(w4a8_quant_act_ex(A, it, 4, 64, i8, f, nullptr));
            EXPECT_RUNTIME(w4fp8_quant_act_ex(A, it, 4, 64, b, f, nullptr));
        }
    }
    EXPECT_RUNTIME(w4a8_quant_act(f, 4, 64, i8, f, nullptr));
    EXPECT_RUNTIME(w4fp8_quant_act(f, 4, 64, b, f, nullptr));
    // W4A8 GEMM and its no-allocation twin
    EXPECT_RUNTIME(w4a8_gemm(i8, f, b, b, b, f, A, 0, 16, 64, 256, 64, 0, nullptr, 0, nullptr));
    EXPECT(w4a8_gemm(nullptr, f, b, b, b, f, A, 0, 16, 64, 256, 64, 0, nullptr, 0, nullptr), W4A8_ERR_NULL_PTR);
    EXPECT(w4a8_gemm(i8, f, b, b, b, f, A, 7, 16, 64, 256, 64, 0, nullptr, 0, nullptr), W4A8_ERR_UNSUPPORTED);
    EXPECT(w4a8_gemm(i8, f, b, b, b, f, A, 0, 16, 64, 256, 64, 3, nullptr, 0, nullptr), W4A8_ERR_SHAPE);
    EXPECT(w4a8_gemm(i8, f, b, mis, b, f, A, 0, 16, 64, 256, 64, 0, nullptr, 0, nullptr), W4A8_ERR_ALIGNMENT);
    EXPECT(w4a8_gemm(i8, f, b, b, b, f, A, 0, 1 << 20, 256, 4096, 64, 0, nullptr, 0, nullptr), W4A8_ERR_SHAPE);
    const size_t need = w4a8_workspace_size(128, 512, 8192, 0);
    if (need == 0) ++fails;
    EXPECT(w4a8_gemm(i8, f, b, b, b, f, A, 0, 128, 512, 8192, 128, 0, A, need - 1, nullptr), W4A8_ERR_WORKSPACE);
    EXPECT(w4a8_gemm(i8, f, b, b, b, f, A, 0, 128, 512, 8192, 128, 0, nullptr, need, nullptr), W4A8_ERR_NULL_PTR);
    EXPECT_RUNTIME(w4a8_gemm(i8, f, b, b, b, f, A, 0, 128, 512, 8192, 128, 0, A, need, nullptr));
    EXPECT_RUNTIME(w4a8_gemm(i8, f, b, b, b, f, A, 1, 16, 64, 256, 64, 2, nullptr, 0, nullptr));
    EXPECT(w4a8_gemm_noalloc(nullptr, f, b, b, b, f, A, 0, 16, 64, 256, 64, 0, nullptr), W4A8_ERR_NULL_PTR);
    EXPECT(w4a8_gemm_noalloc(i8, f, b, b, b, f, A, 0, 16, 64, 200, 64, 0, nullptr), W4A8_ERR_SHAPE);
    EXPECT_RUNTIME(w4a8_gemm_noalloc(i8, f, b, b, b, f, A, 0, 128, 512, 8192, 128, 0, nullptr));
    // grouped, ablation
    EXPECT(w4a8_gemm_grouped(i8, f, i32, 0, b, b, b, f, A, 0, 64, 256, 512, 64, 16, nullptr), W4A8_ERR_SHAPE);
    EXPECT(w4a8_gemm_grouped(i8, f, nullptr, 4, b, b, b, f, A, 0, 64, 256, 512, 64, 16, nullptr), W4A8_ERR_NULL_PTR);
    EXPECT_RUNTIME(w4a8_gemm_grouped(i8, f, i32, 4, b, b, b, f, A, 0, 64, 256, 512, 64, 16, nullptr));
    EXPECT_RUNTIME(w4a8_gemm_grouped(i8, f, i32, 4, b, b, b, f, A, 1, 4096, 256, 512, 64, 1024, nullptr));
    EXPECT(w4a8_gemm_ablation(5, i8, f, b, b, b, f, A, 0, 256, 256, 512, 128, nullptr), W4A8_ERR_UNSUPPORTED);
    EXPECT(w4a8_gemm_ablation(1, i8, f, b, b, b, f, A, 0, 16, 256, 512, 128, nullptr), W4A8_ERR_UNSUPPORTED);
    EXPECT_RUNTIME(w4a8_gemm_ablation(2, i8, f, b, b, b, f, A, 0, 256, 256, 512, 128, nullptr));
    // FP8 variants, folded pack, W8A8
    EXPECT(w4fp8_gemm(b, f, b, f, A, 2, 16, 64, 256, 0, nullptr, 0, nullptr), W4A8_ERR_UNSUPPORTED);
    EXPECT(w4fp8_gemm(b, nullptr, b, f, A, 0, 16, 64, 256, 0, nullptr, 0, nullptr), W4A8_ERR_NULL_PTR);
    EXPECT_RUNTIME(w4fp8_gemm(b, f, b, f, A, 0, 128, 512, 8192, 0, A, need, nullptr));
    EXPECT(w4fp8g_pack(f, 64, 256, 32, b, f, f, nullptr), W4A8_ERR_SHAPE);
    EXPECT_RUNTIME(w4fp8g_pack(f, 64, 256, 64, b, f, f, nullptr));
    EXPECT(w4fp8g_gemm(b, f, b, f, f, A, 0, 16, 256, 512, 96, 0, nullptr, 0, nullptr), W4A8_ERR_SHAPE);
    EXPECT_RUNTIME(w4fp8g_gemm(b, f, b, f, f, A, 1, 16, 256, 512, 64, 0, nullptr, 0, nullptr));
    EXPECT(w8a8_pack(f, 64, 100, i8, f, nullptr), W4A8_ERR_SHAPE);
    EXPECT_RUNTIME(w8a8_pack(f, 64, 256, i8, f, nullptr));
    const size_t need8 = w4a8_workspace_size(128, 256, 8192, 0);
    if (need8 == 0) ++fails;
    EXPECT(w8a8_gemm(i8, f, i8, f, A, 0, 128, 256, 8192, 0, A, need8 - 1, nullptr), W4A8_ERR_WORKSPACE);
    EXPECT_RUNTIME(w8a8_gemm(i8, f, i8, f, A, 0, 16, 256, 512, 0, nullptr, 0, nullptr));

    std::printf("abi driver: %d failures, workspace bytes summed %zu\n", fails, total);
    return fails ? 1 : 0;
}
