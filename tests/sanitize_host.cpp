// Host-side checks of librmm's C ABI, built and run with AddressSanitizer and
// UndefinedBehaviorSanitizer on the library's host code and on this driver
// (tests/test_sanitizers.py).  Only calls that return before any GPU work:
// rmm_k, status strings, descriptor set-up, workspace sizing, plan queries and
// the argument checks of every entry point (fake, aligned device pointers
// that are never dereferenced).  Prints "ok" and exits 0 when every check
// holds; a sanitizer report ends the process with a non-zero status first.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "rmm.h"

static int g_fail = 0;
#define CHECK(cond)                                                    \
    do {                                                               \
        if (!(cond)) {                                                 \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++g_fail;                                                  \
        }                                                              \
    } while (0)

static void *fake(uintptr_t a) { return reinterpret_cast<void *>(a); }

int main() {
    const size_t bad = std::numeric_limits<size_t>::max();

    // k = ceil(rho d), invalid rho or d -> 0
    CHECK(rmm_k(0.8, 4096) == 3277);
    CHECK(rmm_k(0.07, 100) == 7);
    CHECK(rmm_k(1.0, 1) == 1);
    CHECK(rmm_k(0.0, 10) == 0);
    CHECK(rmm_k(1.5, 10) == 0);
    CHECK(rmm_k(std::nan(""), 10) == 0);
    CHECK(rmm_k(0.5, 0) == 0);
    CHECK(rmm_k(0.5, -3) == 0);

    // every int is a valid status argument
    for (int s = -5; s < 12; ++s) CHECK(rmm_status_string(static_cast<rmm_status_t>(s)) != nullptr);
    CHECK(rmm_version() > 0);

    // descriptors, workspace sizes and plans
    rmm_desc_t ds;
    rmm_desc_init(&ds, RMM_BF16, 4096, 4096, 4096);
    const size_t big = rmm_workspace_size(&ds, 0.5);
    CHECK(big > 0 && big < (size_t(1) << 31));
    CHECK(rmm_workspace_size(&ds, 0.0) == bad);
    CHECK(rmm_workspace_size(&ds, std::nan("")) == bad);
    CHECK(rmm_workspace_size(nullptr, 0.5) == bad);
    ds.lda = 100;
    CHECK(rmm_workspace_size(&ds, 0.5) == bad);
    ds.lda = 4096;
    rmm_desc_t odd;
    rmm_desc_init(&odd, static_cast<rmm_dtype_t>(7), 64, 64, 64);  // an unknown dtype code
    CHECK(rmm_workspace_size(&odd, 0.5) == bad);
    rmm_desc_init(&odd, RMM_BF16, 0, 64, 64);
    CHECK(rmm_workspace_size(&odd, 0.5) == bad);
    rmm_desc_init(&odd, RMM_BF16, 64, int64_t(1) << 40, 64);
    CHECK(rmm_workspace_size(&odd, 0.5) == bad);
    const int64_t shapes[][3] = {{4096, 4096, 4096}, {2048, 14336, 4096}, {4096, 8192, 28672}, {1, 8192, 28672},
                                 {1, 8192, 4096},    {300, 520, 40},      {4100, 4096, 4096},  {64, 20480, 64},
                                 {5, 37, 13},        {1, 1, 1}};
    const double rhos[] = {1.0 / 4096, 0.3, 0.5, 0.8, 1.0};
    for (const auto &sh : shapes)
        for (double rho : rhos)
            for (int dt = 0; dt < 2; ++dt) {
                rmm_desc_t q;
                rmm_desc_init(&q, static_cast<rmm_dtype_t>(dt), sh[0], sh[1], sh[2]);
                int32_t info[3] = {-7, -7, -7};
                CHECK(rmm_plan_info(&q, rho, info) == RMM_OK);
                CHECK(info[0] >= 0 && info[2] >= 1);
                const size_t ws = rmm_workspace_size(&q, rho);
                CHECK(ws != bad);
                const int64_t k = rmm_k(rho, sh[1]);
                CHECK(rmm_workspace_size_indexed(&q, k) != bad);
            }
    int32_t info[3];
    CHECK(rmm_plan_info(&ds, 0.5, nullptr) == RMM_ERR_INVALID_ARG);
    CHECK(rmm_plan_info(&ds, 0.0, info) == RMM_ERR_INVALID_ARG);

    // argument errors return before any HIP call
    void *A = fake(uintptr_t(1) << 40), *B = fake(uintptr_t(2) << 40), *Y = fake(uintptr_t(3) << 40);
    char *W = static_cast<char *>(fake(uintptr_t(4) << 40));
    CHECK(rmm_matmul(&ds, nullptr, nullptr, 0.5, nullptr, nullptr, nullptr, 0, nullptr) == RMM_ERR_INVALID_ARG);
    CHECK(rmm_matmul(nullptr, A, B, 0.5, Y, nullptr, nullptr, 0, nullptr) == RMM_ERR_INVALID_ARG);
    CHECK(rmm_select(nullptr, 1, 10, 3, nullptr, nullptr) == RMM_ERR_INVALID_ARG);
    CHECK(rmm_colnorm(nullptr, RMM_BF16, 1, 2, 2, nullptr, nullptr, 0, nullptr) == RMM_ERR_INVALID_ARG);
    rmm_desc_init(&ds, RMM_BF16, 64, 256, 128);
    const size_t need = rmm_workspace_size(&ds, 0.5);
    CHECK(rmm_matmul(&ds, A, B, 0.5, Y, nullptr, W + 16, need, nullptr) == RMM_ERR_INVALID_ARG);
    CHECK(rmm_matmul(&ds, A, B, 0.5, Y, nullptr, W, need - 1, nullptr) == RMM_ERR_WORKSPACE);
    CHECK(rmm_matmul_noalloc(&ds, A, B, std::nan(""), Y, nullptr, nullptr) == RMM_ERR_INVALID_ARG);
    const int32_t *I = static_cast<const int32_t *>(fake(uintptr_t(5) << 40));
    const size_t need_i = rmm_workspace_size_indexed(&ds, 128);
    CHECK(rmm_workspace_size_indexed(&ds, 0) == bad);
    CHECK(rmm_workspace_size_indexed(&ds, 257) == bad);
    CHECK(rmm_matmul_indexed(&ds, A, B, nullptr, 128, Y, W, need_i, nullptr) == RMM_ERR_INVALID_ARG);
    CHECK(rmm_matmul_indexed(&ds, A, B, I, 257, Y, W, need_i, nullptr) == RMM_ERR_INVALID_ARG);
    CHECK(rmm_matmul_indexed(&ds, A, B, I, 128, Y, W, need_i - 1, nullptr) == RMM_ERR_WORKSPACE);

    // attention, decode over 8-bit weights, the 8-bit GEMM and the gated block
    CHECK(rmm_attention_workspace_size(32, 8, 4096, 4096, 128, 0.5) != bad);
    CHECK(rmm_attention_workspace_size(32, 6, 64, 64, 128, 0.5) == bad);
    CHECK(rmm_attention_workspace_size(4, 4, 64, 64, 100, 0.5) == bad);
    void *q = fake(0x10000), *kk = fake(0x20000), *v = fake(0x30000), *o = fake(0x40000), *w = fake(0x100000);
    const size_t need_a = rmm_attention_workspace_size(2, 1, 64, 64, 128, 0.5);
    CHECK(rmm_attention(nullptr, kk, v, 2, 1, 64, 64, 128, 128, 0.5, 1, o, nullptr, w, need_a, nullptr) ==
          RMM_ERR_INVALID_ARG);
    CHECK(rmm_attention(q, kk, v, 2, 1, 64, 64, 128, 128, 0.5, 2, o, nullptr, w, need_a, nullptr) ==
          RMM_ERR_INVALID_ARG);
    CHECK(rmm_attention(q, kk, v, 2, 1, 64, 64, 128, 128, 0.5, 1, o, nullptr, w, need_a - 1, nullptr) ==
          RMM_ERR_WORKSPACE);
    CHECK(rmm_decode_wq_workspace_size(8192, 28672, 0.8) != bad);
    CHECK(rmm_decode_wq_workspace_size(8192, 40, 0.8) == bad);
    const size_t need_d = rmm_decode_wq_workspace_size(1024, 256, 0.5);
    const float *sc = static_cast<const float *>(fake(0x30000));
    CHECK(rmm_decode_wq(fake(0x10000), fake(0x200000), 2, sc, 1024, 256, 256, 0.5, 1.f, fake(0x40000), nullptr, w,
                        need_d, nullptr) == RMM_ERR_INVALID_ARG);
    CHECK(rmm_decode_wq(fake(0x10000), fake(0x200000), 0, sc, 1024, 256, 256, 0.5, 1.f, fake(0x40000), nullptr, w,
                        need_d - 1, nullptr) == RMM_ERR_WORKSPACE);
    CHECK(rmm_matmul_wq_workspace_size(4096, 8192, 28672, 0.8) != bad);
    CHECK(rmm_matmul_wq_workspace_size(4096, 8192, 28672, 0.0) == bad);
    CHECK(rmm_gated_mlp_workspace_size(2048, 4096, 14336, 0.8, 0.8) != bad);
    CHECK(rmm_gated_mlp_workspace_size(2048, 4096, 14330, 0.8, 0.8) == bad);
    CHECK(rmm_gated_weights(nullptr, nullptr, 4096, 14336, 0, nullptr, nullptr) == RMM_ERR_INVALID_ARG);
    CHECK(rmm_timing_collect(nullptr, nullptr) == RMM_ERR_INVALID_ARG);

    if (g_fail) {
        std::fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
