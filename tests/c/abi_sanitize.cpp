// Drives the C ABI of libqmm (include/qmm.h) on a machine without a GPU, for a build of the
// library's host code with -fsanitize=address,undefined: every argument check, workspace
// layout, planner path and override, plus calls with valid shapes whose launches then fail for
// want of a device (QMM_ERR_HIP).  Pointers passed as device memory are fake addresses that only a
// kernel would dereference -- so the program refuses to run (prints "skip" and exits 0) when any
// GPU is visible.  Exit status 0 and a final "ok": no sanitizer finding and every status as
// expected.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <thread>
#include <vector>

#include "qmm.h"

static int failures = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "line %d: %s (%s)\n", __LINE__, #cond, qmm_last_error()); \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static void *fake(uintptr_t a) { return reinterpret_cast<void *>(a); }

int main() {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
        std::printf("skip: a GPU is visible (%d)\n", ndev);
        return 0;
    }
    const int types[] = {QMM_Q4_0, QMM_Q8_0, QMM_Q4_K, QMM_Q5_K, QMM_Q6_K};
    void *W = fake(0x100000), *X = fake(0x200000), *Y = fake(0x300000), *WS = fake(0x400000);
    const int32_t *IDS = static_cast<const int32_t *>(fake(0x500000));

    // argument errors
    EXPECT(qmm_matmul(3, W, 16, 256, (const float *)X, 1, (float *)Y, WS, 1 << 30, nullptr) == QMM_ERR_TYPE);
    EXPECT(qmm_matmul(QMM_Q4_K, W, 16, 100, (const float *)X, 1, (float *)Y, WS, 1 << 30, nullptr) == QMM_ERR_SHAPE);
    EXPECT(qmm_matmul(QMM_Q4_K, W, 0, 256, (const float *)X, 1, (float *)Y, WS, 1 << 30, nullptr) == QMM_ERR_ARG);
    EXPECT(qmm_matmul(QMM_Q4_K, W, 16, 256, (const float *)X, -1, (float *)Y, WS, 1 << 30, nullptr) == QMM_ERR_ARG);
    EXPECT(qmm_matmul(QMM_Q4_K, fake(0x100001), 16, 256, (const float *)X, 1, (float *)Y, WS, 1 << 30, nullptr) ==
           QMM_ERR_ARG);
    EXPECT(qmm_matmul(QMM_Q4_K, W, 16, 256, (const float *)fake(0x200004), 1, (float *)Y, WS, 1 << 30, nullptr) ==
           QMM_ERR_ARG);
    EXPECT(qmm_matmul(QMM_Q4_K, W, 16, 256, (const float *)X, 0, nullptr, nullptr, 0, nullptr) == QMM_OK);
    EXPECT(qmm_matmul(QMM_Q4_K, W, 4096, 4096, (const float *)X, 512, (float *)Y, WS, 16, nullptr) ==
           QMM_ERR_WORKSPACE);
    EXPECT(qmm_matmul(QMM_Q4_K, W, 16, (int64_t)1 << 21, (const float *)X, 1, (float *)Y, WS, 0, nullptr) ==
           QMM_ERR_SHAPE);
    EXPECT(qmm_quantize_q8_1((const float *)X, 1, 33, Y, nullptr) == QMM_ERR_SHAPE);
    EXPECT(qmm_matmul_id(QMM_Q4_K, W, 4, 16, 256, (const float *)X, 3, IDS, 8, 2, (float *)Y, WS, 1 << 30,
                         nullptr) == QMM_ERR_ARG);
    EXPECT(qmm_matmul_id(QMM_Q4_K, W, 0, 16, 256, (const float *)X, 1, IDS, 8, 2, (float *)Y, WS, 1 << 30,
                         nullptr) == QMM_ERR_ARG);
    EXPECT(qmm_matmul_glu(QMM_Q4_K, W, nullptr, 16, 256, (const float *)X, 1, (float *)Y, WS, 1 << 30, nullptr) ==
           QMM_ERR_ARG);
    EXPECT(qmm_matmul_f16act(QMM_Q4_K, W, 16, 256, (const float *)X, 9, (float *)Y, WS, 1 << 30, nullptr) ==
           QMM_ERR_ARG);
    EXPECT(qmm_debug_subdots(QMM_Q4_K, W, 16, 256, X, 1, 3, (int32_t *)Y, WS, 1 << 30, nullptr) == QMM_ERR_ARG);
    EXPECT(qmm_debug_subdots(QMM_Q4_K, W, 16, 256, X, 40, 2, (int32_t *)Y, WS, 16, nullptr) == QMM_ERR_WORKSPACE);
    EXPECT(qmm_set_override(99, 1) == QMM_ERR_ARG);
    EXPECT(qmm_set_override(QMM_OVR_TILE_J, 48) == QMM_ERR_ARG);

    // planner, workspace sizes and kernel choices over many shapes (host logic only)
    const int64_t ks[] = {256, 512, 4096, 14336, 32768, 33024};
    const int64_t ns[] = {0, 1, 2, 5, 8, 9, 16, 100, 512, 2048};
    for (int t : types)
        for (int64_t k : ks)
            for (int64_t n : ns) {
                qmm_plan p{};
                const qmm_status st = qmm_plan_dense(t, 4096, k, n, 256, &p);
                EXPECT(st == QMM_OK);
                EXPECT(p.ws_bytes == qmm_matmul_workspace(t, 4096, k, n));
                (void)qmm_matmul_q8_1_workspace(t, 4096, k, n);
                (void)qmm_matmul_glu_workspace(t, 4096, k, n);
                (void)qmm_debug_subdots_workspace(t, 100, k, n, 2);
                int32_t kid = -1;
                if (n >= 1) EXPECT(qmm_matvec_kernel(t, W, 4096, k, X, n, 1, &kid) == QMM_OK);
                int64_t lay[6];
                EXPECT(qmm_matmul_id_grouping_layout(t, 128, k, n, 8, 1, lay) == QMM_OK);
                (void)qmm_matmul_id_workspace(t, 128, 768, k, n, 8, 8);
                (void)qmm_matmul_f16act_workspace(k, n);
            }
    EXPECT(qmm_tile_efficiency(100, 108) == 92 && qmm_tile_efficiency(120, 108) == 55);
    EXPECT(qmm_streamk_unit_start(3, 7, 5, 9) == (3 * 45) / 7);

    // valid calls: everything up to the launch runs, the launch fails without a device
    for (int t : types) {
        const int64_t k = 4096;
        for (int64_t n : {1, 3, 8, 40, 512}) {
            const size_t ws = qmm_matmul_workspace(t, 4096, k, n);
            EXPECT(qmm_matmul(t, W, 4096, k, (const float *)X, n, (float *)Y, WS, ws, nullptr) == QMM_ERR_HIP);
            const size_t wq = qmm_matmul_q8_1_workspace(t, 4096, k, n);
            EXPECT(qmm_matmul_q8_1(t, W, 4096, k, X, n, (float *)Y, WS, wq, nullptr) == QMM_ERR_HIP);
            const size_t wg = qmm_matmul_glu_workspace(t, 4096, k, n);
            EXPECT(qmm_matmul_glu(t, W, W, 4096, k, (const float *)X, n, (float *)Y, WS, wg, nullptr) == QMM_ERR_HIP);
            const size_t wd = qmm_debug_subdots_workspace(t, 4096, k, n, 2);
            EXPECT(qmm_debug_subdots(t, W, 4096, k, X, n, 2, (int32_t *)Y, WS, wd, nullptr) == QMM_ERR_HIP);
            if (n <= 8) {
                const size_t wf = qmm_matmul_f16act_workspace(k, n);
                EXPECT(qmm_matmul_f16act(t, W, 4096, k, (const float *)X, n, (float *)Y, WS, wf, nullptr) ==
                       QMM_ERR_HIP);
            }
        }
        const size_t wi = qmm_matmul_id_workspace(t, 128, 768, 2048, 2048, 8, 8);
        EXPECT(qmm_matmul_id(t, W, 128, 768, 2048, (const float *)X, 8, IDS, 2048, 8, (float *)Y, WS, wi, nullptr) ==
               QMM_ERR_HIP);
        const size_t wig = qmm_matmul_id_glu_workspace(t, 128, 768, 2048, 2048, 8);
        EXPECT(qmm_matmul_id_glu(t, W, W, 128, 768, 2048, (const float *)X, IDS, 2048, 8, (float *)Y, WS, wig,
                                 nullptr) == QMM_ERR_HIP);
    }
    int64_t cnt = 0;
    EXPECT(qmm_matmul_id_invalid_count(WS, &cnt, nullptr) == QMM_ERR_HIP);
    // allocation-free entry point: too large for its scratch (host check), argument errors, and a
    // call that fits -- its scratch lookup fails without a device
    EXPECT(qmm_matmul_noalloc(QMM_Q6_K, W, 4096, 14336, (const float *)X, 65536, (float *)Y, nullptr) ==
           QMM_ERR_WORKSPACE);
    EXPECT(qmm_matmul_noalloc(3, W, 4096, 256, (const float *)X, 4, (float *)Y, nullptr) == QMM_ERR_TYPE);
    EXPECT(qmm_matmul_noalloc(QMM_Q4_K, W, 4096, 4096, (const float *)X, 0, (float *)Y, nullptr) == QMM_OK);
    for (int64_t n : {3, 512})
        EXPECT(qmm_matmul_noalloc(QMM_Q4_K, W, 4096, 4096, (const float *)X, n, (float *)Y, nullptr) == QMM_ERR_HIP);

    // overrides written while other threads plan
    std::atomic<bool> stop{false};
    std::thread wr([&] {
        for (int i = 0; !stop.load(); ++i) {
            qmm_set_override(QMM_OVR_PATH, (i & 1) ? 2 : 0);
            qmm_set_override(QMM_OVR_TILE_J, (i % 3) * 32);
            qmm_set_override(QMM_OVR_MV_KERNEL, i % 4);
        }
    });
    std::vector<std::thread> rd;
    std::atomic<int> bad{0};
    for (int r = 0; r < 4; ++r)
        rd.emplace_back([&] {
            for (int i = 0; i < 20000; ++i) {
                qmm_plan p{};
                if (qmm_plan_dense(QMM_Q4_K, 4096, 4096, 4, 256, &p) != QMM_OK) ++bad;
                if (!((p.regime == 1 && p.tile_j == 8) || (p.regime == 2 && p.tile_j >= 32))) ++bad;
            }
        });
    for (auto &t : rd) t.join();
    stop = true;
    wr.join();
    EXPECT(bad.load() == 0);
    for (int key = 1; key <= 6; ++key) qmm_set_override(key, 0);

    if (failures) return 1;
    std::printf("ok\n");
    return 0;
}
