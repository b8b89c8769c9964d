// oracle_check.cpp -- drives every entry point of the CPU oracle
// (oracle/oracle.cpp) over special values, odd sizes, strided rows and more
// threads than elements, for an AddressSanitizer + UndefinedBehaviorSanitizer
// build (tests/test_sanitizers.py). Any sanitizer report aborts the program;
// otherwise it checks a few plain facts and prints "ok".
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <limits>
#include <vector>

extern "C" {
void oracle_f32_to_bf16(const float*, uint16_t*, int64_t);
void oracle_bf16_to_f32(const uint16_t*, float*, int64_t);
void oracle_gelu_tanh_f64(const double*, double*, int64_t);
void oracle_gelu_tanh_literal_f64(const double*, double*, int64_t);
void oracle_gelu_tanh_f32(const float*, float*, int64_t, int);
void oracle_gelu_tanh_bf16(const uint16_t*, uint16_t*, int64_t, int);
int oracle_chain_f32(const float*, float*, int64_t, const int32_t*, const float*, int, int);
int oracle_chain_bf16(const uint16_t*, uint16_t*, int64_t, const int32_t*, const float*, int, int);
int oracle_softmax_rows_f64(const double*, double*, int64_t, int64_t, int64_t, int64_t);
int oracle_softmax_rows_f32(const float*, float*, int64_t, int64_t, int64_t, int64_t, int);
int oracle_softmax_rows_bf16(const uint16_t*, uint16_t*, int64_t, int64_t, int64_t, int64_t, int);
void oracle_gelu_tanh_grad_f64(const double*, double*, int64_t);
void oracle_gelu_tanh_bwd_f32(const float*, const float*, float*, int64_t, int);
void oracle_gelu_tanh_bwd_bf16(const uint16_t*, const uint16_t*, uint16_t*, int64_t, int);
int oracle_softmax_bwd_rows_f64(const double*, const double*, double*, int64_t, int64_t);
int oracle_softmax_bwd_rows_f32(const float*, const float*, float*, int64_t, int64_t, int);
int oracle_softmax_bwd_rows_bf16(const uint16_t*, const uint16_t*, uint16_t*, int64_t, int64_t, int);
int oracle_layernorm_rows_f64(const double*, double*, int64_t, int64_t, int64_t, int64_t,
                              const double*, const double*, double, int);
int oracle_layernorm_rows_f32(const float*, float*, int64_t, int64_t, int64_t, int64_t,
                              const float*, const float*, double, int, int);
int oracle_layernorm_rows_bf16(const uint16_t*, uint16_t*, int64_t, int64_t, int64_t, int64_t,
                               const uint16_t*, const uint16_t*, double, int, int);
}

static int failures = 0;
#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            std::printf("failed: %s (line %d)\n", #c, __LINE__);   \
            ++failures;                                            \
        }                                                          \
    } while (0)

int main() {
    const float inf = std::numeric_limits<float>::infinity();
    const float nan = std::numeric_limits<float>::quiet_NaN();
    std::vector<float> f = {0.0f, -0.0f, 1.0f, -1.0f, 3.5f, -9.5f, -30.0f, 1e-40f, -1e-40f,
                            3e38f, -3e38f, inf, -inf, nan, 6.0f, -6.0f, 0.25f};
    const int64_t n = static_cast<int64_t>(f.size());
    std::vector<double> d(f.begin(), f.end()), dy(n);
    std::vector<uint16_t> b(n), b2(n);
    std::vector<float> y(n), g(n);

    oracle_f32_to_bf16(f.data(), b.data(), n);
    oracle_bf16_to_f32(b.data(), y.data(), n);
    oracle_gelu_tanh_f64(d.data(), dy.data(), n);
    oracle_gelu_tanh_literal_f64(d.data(), dy.data(), n);
    oracle_gelu_tanh_grad_f64(d.data(), dy.data(), n);
    for (int t : {1, 3, 64}) {  // more threads than elements too
        oracle_gelu_tanh_f32(f.data(), y.data(), n, t);
        oracle_gelu_tanh_bf16(b.data(), b2.data(), n, t);
        oracle_gelu_tanh_bwd_f32(f.data(), f.data(), g.data(), n, t);
        oracle_gelu_tanh_bwd_bf16(b.data(), b.data(), b2.data(), n, t);
    }
    oracle_gelu_tanh_f32(f.data(), y.data(), 0, 4);  // empty
    CHECK(y[0] == 0.0f && !std::signbit(y[0]));

    const int32_t kinds[4] = {1, 3, 2, 4};
    const float scal[4] = {1.0f, 0.0f, 0.5f, 0.0f};
    CHECK(oracle_chain_f32(f.data(), y.data(), n, kinds, scal, 4, 2) == 0);
    CHECK(oracle_chain_bf16(b.data(), b2.data(), n, kinds, scal, 4, 2) == 0);
    const int32_t bad[1] = {9};
    CHECK(oracle_chain_f32(f.data(), y.data(), n, bad, scal, 1, 1) == -1);
    CHECK(oracle_chain_f32(f.data(), y.data(), n, kinds, scal, 0, 1) == -1);

    // rows of 5 columns, stride 7 (the padding untouched), specials in some rows
    const int64_t rows = 4, cols = 5, ld = 7;
    std::vector<float> xs(rows * ld, 0.5f), ys(rows * ld, 123.0f);
    xs[0] = inf;              // row 0 -> NaN
    xs[ld + 2] = nan;         // row 1 -> NaN
    for (int64_t j = 0; j < cols; ++j) xs[2 * ld + j] = -inf;  // row 2 -> NaN
    xs[3 * ld + 1] = 80.0f;
    std::vector<double> xd(xs.begin(), xs.end()), yd(rows * ld, 0.0);
    std::vector<uint16_t> xb(rows * ld), yb(rows * ld);
    oracle_f32_to_bf16(xs.data(), xb.data(), rows * ld);
    CHECK(oracle_softmax_rows_f64(xd.data(), yd.data(), rows, cols, ld, ld) == 0);
    CHECK(oracle_softmax_rows_f32(xs.data(), ys.data(), rows, cols, ld, ld, 3) == 0);
    CHECK(oracle_softmax_rows_bf16(xb.data(), yb.data(), rows, cols, ld, ld, 8) == 0);
    CHECK(ys[5] == 123.0f && ys[6] == 123.0f);  // stride padding untouched
    CHECK(std::isnan(ys[0]) && std::isnan(ys[ld]) && std::isnan(ys[2 * ld]));
    CHECK(oracle_softmax_rows_f32(xs.data(), ys.data(), rows, cols, cols - 1, ld, 1) == -1);
    CHECK(oracle_softmax_rows_f32(xs.data(), ys.data(), -1, cols, ld, ld, 1) == -1);
    CHECK(oracle_softmax_rows_f32(nullptr, nullptr, 0, cols, ld, ld, 1) == 0);

    std::vector<double> gy(rows * cols, 0.2), gdy(rows * cols, 1.0), gdx(rows * cols);
    std::vector<float> fy(rows * cols, 0.2f), fdy(rows * cols, -1.0f), fdx(rows * cols);
    std::vector<uint16_t> by(rows * cols), bdy(rows * cols), bdx(rows * cols);
    oracle_f32_to_bf16(fy.data(), by.data(), rows * cols);
    oracle_f32_to_bf16(fdy.data(), bdy.data(), rows * cols);
    CHECK(oracle_softmax_bwd_rows_f64(gy.data(), gdy.data(), gdx.data(), rows, cols) == 0);
    CHECK(oracle_softmax_bwd_rows_f32(fy.data(), fdy.data(), fdx.data(), rows, cols, 5) == 0);
    CHECK(oracle_softmax_bwd_rows_bf16(by.data(), bdy.data(), bdx.data(), rows, cols, 2) == 0);
    CHECK(oracle_softmax_bwd_rows_f32(nullptr, fdy.data(), fdx.data(), rows, cols, 1) == -1);

    std::vector<double> gam(cols, 1.5), bet(cols, -0.25);
    std::vector<float> gamf(cols, 1.5f), betf(cols, -0.25f);
    std::vector<uint16_t> gamb(cols), betb(cols);
    oracle_f32_to_bf16(gamf.data(), gamb.data(), cols);
    oracle_f32_to_bf16(betf.data(), betb.data(), cols);
    for (int gelu : {0, 1}) {
        CHECK(oracle_layernorm_rows_f64(xd.data(), yd.data(), rows, cols, ld, ld, gam.data(),
                                        bet.data(), 1e-5, gelu) == 0);
        CHECK(oracle_layernorm_rows_f32(xs.data(), ys.data(), rows, cols, ld, ld, gamf.data(),
                                        betf.data(), 1e-5, gelu, 4) == 0);
        CHECK(oracle_layernorm_rows_bf16(xb.data(), yb.data(), rows, cols, ld, ld, nullptr,
                                         nullptr, 0.0, gelu, 1) == 0);
    }
    CHECK(oracle_layernorm_rows_f32(xs.data(), ys.data(), rows, cols, ld, ld, nullptr, nullptr,
                                    -1.0, 0, 1) == -1);
    if (failures) return 1;
    std::printf("ok\n");
    return 0;
}
