// api_check.cpp -- drives the host-side argument checks of every libfusedops
// entry point with extreme sizes, strides and pointers, for a build whose
// host code carries AddressSanitizer + UndefinedBehaviorSanitizer
// (tests/test_sanitizers.py). Every call here is refused (or has no work)
// before any HIP call, so no GPU is needed; a signed overflow in the size
// arithmetic, or any memory error, aborts the program. Prints "ok".
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <limits>

#include "fusedops.h"

static int failures = 0;
#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            std::printf("failed: %s (line %d)\n", #c, __LINE__);   \
            ++failures;                                            \
        }                                                          \
    } while (0)

int main() {
    const int64_t M = std::numeric_limits<int64_t>::max();
    const int64_t m = std::numeric_limits<int64_t>::min();
    char* a = reinterpret_cast<char*>(uintptr_t(0x7F0000000000ull));
    char* b = reinterpret_cast<char*>(uintptr_t(0x7F8000000000ull));
    char* c = reinterpret_cast<char*>(uintptr_t(0x7FC000000000ull));
    const int64_t sizes[] = {-1, m, M, M / 2, M / 4 + 1, int64_t(1) << 62, int64_t(1) << 40};
    const int all_dtypes[] = {FK_F32, FK_BF16, FK_F16, 7, -3};
    const int row_dtypes[] = {FK_F32, FK_BF16};
    fk_op ops[FK_MAX_OPS];
    for (auto& o : ops) o = fk_op{FK_OP_ADD_SCALAR, 1.0f};

    for (int64_t n : sizes) {
        for (int dt : all_dtypes) {
            const int r1 = fk_gelu_tanh(a, b, n, dt, nullptr);
            const int r2 = fk_elementwise_chain(a, b, n, dt, ops, FK_MAX_OPS, nullptr);
            const int r3 = fk_gelu_tanh_backward(a, b, c, n, dt, nullptr);
            CHECK(r1 < 0 && r2 < 0 && r3 < 0);
        }
        CHECK(fk_copy(a, b, n, nullptr) < 0);
        for (int64_t k : sizes) {
            for (int dt : row_dtypes) {
                CHECK(fk_softmax_rows(a, b, n, k, k, k, dt, nullptr) < 0);
                CHECK(fk_softmax_rows_online(a, b, n, k, k, k, dt, nullptr) < 0);
                CHECK(fk_softmax_rows_noalloc(a, b, n, k, k, k, dt, nullptr) < 0);
                CHECK(fk_softmax_rows_ws(a, b, n, k, k, k, dt, c, M, nullptr) < 0);
                CHECK(fk_softmax_rows_path(a, b, n, k, k, k, dt, M) < 0);
                CHECK(fk_layernorm_rows(a, b, n, k, k, k, nullptr, nullptr, 1e-5f, 1, dt,
                                        nullptr) < 0);
                CHECK(fk_softmax_rows_backward(a, b, c, n, k, k, k, k, dt, nullptr) < 0);
                const int64_t w = fk_softmax_workspace_bytes(n, k, dt);
                CHECK(w == FK_ERR_INVALID_ARG || w >= 0);
            }
            CHECK(fk_linear_gelu(a, b, nullptr, c, n, k, k, k, k, k, FK_ACT_GELU_TANH, FK_BF16,
                                 nullptr) < 0);
            int64_t st[12];
            for (int i = 0; i < 12; ++i) st[i] = k;
            CHECK(fk_attention_fwd(a, b, c, c, n, k, k, 128, st, 1, FK_BF16, nullptr) < 0);
            CHECK(fk_attention_fwd(a, b, c, c, 1, 1, n, 128, st, 0, FK_F16, nullptr) < 0);
        }
    }
    // queries and settings
    CHECK(fk_softmax_onchip_max_cols(FK_F32) > 0 && fk_softmax_onchip_max_cols(9) < 0);
    CHECK(fk_layernorm_max_cols(FK_BF16) > 0 && fk_softmax_backward_max_cols(FK_F16) < 0);
    CHECK(fk_set_split_wait_limit(-5) == FK_ERR_INVALID_ARG);
    const int64_t prev = fk_set_split_wait_limit(M);
    CHECK(fk_set_split_wait_limit(prev) == M);
    for (int s = -10; s <= 10; ++s) CHECK(fk_status_string(s) != nullptr);
    // empty work
    CHECK(fk_gelu_tanh(nullptr, nullptr, 0, FK_F32, nullptr) == FK_OK);
    CHECK(fk_softmax_rows_noalloc(nullptr, nullptr, 0, 5, 5, 5, FK_F32, nullptr) == FK_OK);
    CHECK(fk_softmax_rows_path(nullptr, nullptr, 3, 0, 0, 0, FK_BF16, 0) == FK_PATH_NONE);
    if (failures) return 1;
    std::printf("ok\n");
    return 0;
}
