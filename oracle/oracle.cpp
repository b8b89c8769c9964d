// oracle.cpp -- plain, slow CPU oracle for the fused memory-bound kernels.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
// call this file: only the tests, the smoke check and the benchmark's CPU
// baseline leg use it. It shares no code, header, table or constant
// generator with the HIP library; it is built on its own with g++.
//
// Every result is computed from its plain definition in double precision
// and rounded once to the storage type (fp32, or fp32 then bf16). There is
// no blocking, fusion, vectorisation or reordering: one element, or one row,
// at a time in index order. The optional thread count only splits the index
// range (or the row range) into contiguous independent pieces, so results do
// not depend on it.
//
// Sources (web pages on GPU kernels and fusion):
//  * GELU: "CS336 lecture 6" study notes (kyc001.github.io), section 4.2,
//    "Case: GELU" -- GELU(x) ~= 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).
//    The tanh form is the definition used here.
//  * Row softmax: same notes, section 5.2 -- per row: load the row, take
//    its max, take exponentials and their sum, normalise and write back;
//    and "Lecture 6: GPU Kernels and Triton" (cs336.sjfarmltd.com),
//    section 7.2 "Online Softmax" -- the standard softmax subtracts the row
//    max for stability and divides exp(x - max) by the sum.
//  * Chain: "Lecture 6: GPU Kernels and Triton", section 1.1 (three
//    consecutive elementwise ops) -- each op is applied in order and each
//    intermediate is materialised in the I/O compute type (fp32).
//  * LayerNorm: "Lecture 6: GPU Kernels and Triton", section 6.1 names it as
//    the first kernel of the LayerNorm -> Linear -> GELU example without a
//    formula; the standard definition over the last axis is used: mean, the
//    biased variance, (x - mean) / sqrt(var + eps), then gamma and beta per
//    column, optionally followed by the tanh-GELU above.
//  * Backward (the pages print no formulas; the Triton tutorial page,
//    accesspath.com "Triton in practice", names autograd integration as
//    later work): derived from the forward definitions above.
//    GELU'(x) = s + 2 x k (1 + 3 c x^2) s (1 - s), s = 1 / (1 + e^(-2u)),
//    k = sqrt(2/pi), c = 0.044715, with 1 - s evaluated as 1 / (1 + e^(2u));
//    dx = dy * GELU'(x). Softmax: dx_j = y_j (dy_j - sum_k y_k dy_k), the
//    Jacobian-vector product of y = softmax(x).
//
// Readings where the pages are silent (each also listed in the design notes):
//  * GELU(-inf) = -0 (the limit), GELU(NaN) = NaN, GELU(+inf) = +inf.
//  * bf16 rounding is round-to-nearest-even; NaN stays NaN (quiet).
//  * A softmax row holding NaN or +inf, or only -inf, becomes all NaN
//    (what the formula gives).
//
// Pins: tests/test_oracle_*.py check this file against torch's and scipy's
// own routines, the definitions evaluated exactly in high-precision decimal
// arithmetic, closed-form identities and the pages' worked example.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------- bf16 ----
// bf16 is the upper half of an IEEE binary32 pattern.
float bf16_to_f32(uint16_t b) {
    uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    std::memcpy(&f, &u, sizeof f);
    return f;
}

// Round a binary32 value to bf16, nearest with ties to even.
uint16_t f32_to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, sizeof u);
    if (std::isnan(f)) {
        // keep sign and leading payload bits, set the quiet bit
        return static_cast<uint16_t>((u >> 16) | 0x0040u);
    }
    uint32_t upper = u >> 16;      // the kept half
    uint32_t lower = u & 0xFFFFu;  // the discarded half
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) {
        upper += 1;  // a carry into the exponent is correct (max finite -> inf)
    }
    return static_cast<uint16_t>(upper);
}

// ---------------------------------------------------------------- GELU ----
const double kSqrt2OverPi = std::sqrt(2.0 / M_PI);
const double kCubic = 0.044715;

// u = sqrt(2/pi) * (x + 0.044715 x^3), the tanh argument.
double gelu_u(double x) { return kSqrt2OverPi * (x + kCubic * x * x * x); }

// The literal formula of the notes: 0.5 x (1 + tanh u).
// Loses relative accuracy for very negative x (1 + tanh u cancels).
double gelu_literal(double x) { return 0.5 * x * (1.0 + std::tanh(gelu_u(x))); }

// The same real function, written without the cancellation:
// 1 + tanh u = 2 / (1 + exp(-2u)), so 0.5 x (1 + tanh u) = x / (1 + exp(-2u)).
double gelu_real(double x) {
    if (std::isnan(x)) return x;
    if (x == -std::numeric_limits<double>::infinity()) return -0.0;  // the limit
    return x / (1.0 + std::exp(-2.0 * gelu_u(x)));
}

// Derivative of the real tanh-GELU. Limits at +-inf (1 and 0); where
// s (1 - s) underflows the second term is 0 (it avoids 0 * inf).
double gelu_grad_real(double x) {
    if (std::isnan(x)) return x;
    if (x == std::numeric_limits<double>::infinity()) return 1.0;
    if (x == -std::numeric_limits<double>::infinity()) return 0.0;
    const double u = gelu_u(x);
    const double s = 1.0 / (1.0 + std::exp(-2.0 * u));
    const double q = 1.0 / (1.0 + std::exp(2.0 * u));  // 1 - s
    const double sq = s * q;
    if (sq == 0.0) return s;
    const double du = kSqrt2OverPi * (1.0 + 3.0 * kCubic * x * x);
    return s + 2.0 * x * du * sq;
}

// ---------------------------------------------------------------- chain ---
enum OpKind { kAdd = 1, kMul = 2, kGelu = 3, kRelu = 4 };

// ReLU: x for x > 0, else +0; NaN stays NaN.
double relu_real(double x) { return (x > 0.0 || std::isnan(x)) ? x : 0.0; }

bool ops_valid(const int32_t* kinds, int n_ops) {
    if (n_ops < 1 || kinds == nullptr) return false;
    for (int i = 0; i < n_ops; ++i)
        if (kinds[i] != kAdd && kinds[i] != kMul && kinds[i] != kGelu && kinds[i] != kRelu)
            return false;
    return true;
}

// Apply the ops in order; each op is computed in double and its result is
// rounded to fp32, as if each op were its own kernel writing fp32.
float chain_one(float v, const int32_t* kinds, const float* scalars, int n_ops) {
    for (int i = 0; i < n_ops; ++i) {
        double r = 0.0;
        switch (kinds[i]) {
            case kAdd: r = static_cast<double>(v) + static_cast<double>(scalars[i]); break;
            case kMul: r = static_cast<double>(v) * static_cast<double>(scalars[i]); break;
            case kGelu: r = gelu_real(static_cast<double>(v)); break;
            case kRelu: r = relu_real(static_cast<double>(v)); break;
        }
        v = static_cast<float>(r);
    }
    return v;
}

// ---------------------------------------------------------------- softmax -
// One row, in double: m = max_j x_j; s = sum_j exp(x_j - m); y_j = exp(x_j - m) / s.
void softmax_row(const double* x, double* y, int64_t cols) {
    double m = -std::numeric_limits<double>::infinity();
    for (int64_t j = 0; j < cols; ++j)
        if (x[j] > m) m = x[j];
    double s = 0.0;
    for (int64_t j = 0; j < cols; ++j) s += std::exp(x[j] - m);
    for (int64_t j = 0; j < cols; ++j) y[j] = std::exp(x[j] - m) / s;
}

// ---------------------------------------------------------------- layernorm
// One row in double: mu = sum_j x_j / n; var = sum_j (x_j - mu)^2 / n;
// y_j = (x_j - mu) / sqrt(var + eps) * gamma_j + beta_j (gamma = 1, beta = 0
// when absent), then y_j = GELU(y_j) if requested.
void layernorm_row(const double* x, double* y, int64_t cols, const double* gamma,
                   const double* beta, double eps, bool gelu) {
    double sum = 0.0;
    for (int64_t j = 0; j < cols; ++j) sum += x[j];
    const double mu = sum / static_cast<double>(cols);
    double sq = 0.0;
    for (int64_t j = 0; j < cols; ++j) sq += (x[j] - mu) * (x[j] - mu);
    const double var = sq / static_cast<double>(cols);
    const double denom = std::sqrt(var + eps);
    for (int64_t j = 0; j < cols; ++j) {
        double v = (x[j] - mu) / denom;
        if (gamma != nullptr) v *= gamma[j];
        if (beta != nullptr) v += beta[j];
        y[j] = gelu ? gelu_real(v) : v;
    }
}

// ------------------------------------------------------- softmax backward -
// One row in double: dot = sum_k y_k dy_k; dx_j = y_j (dy_j - dot).
void softmax_bwd_row(const double* y, const double* dy, double* dx, int64_t cols) {
    double dot = 0.0;
    for (int64_t j = 0; j < cols; ++j) dot += y[j] * dy[j];
    for (int64_t j = 0; j < cols; ++j) dx[j] = y[j] * (dy[j] - dot);
}

// ---------------------------------------------------------------- threads -
// Run body(begin, end) over [0, n) split into contiguous pieces.
template <class Body>
void parallel_range(int64_t n, int nthreads, Body body) {
    if (nthreads <= 1 || n < 2) {
        body(int64_t{0}, n);
        return;
    }
    if (static_cast<int64_t>(nthreads) > n) nthreads = static_cast<int>(n);
    std::vector<std::thread> pool;
    pool.reserve(nthreads);
    for (int t = 0; t < nthreads; ++t) {
        int64_t b = n * t / nthreads;
        int64_t e = n * (t + 1) / nthreads;
        pool.emplace_back([=] { body(b, e); });
    }
    for (auto& th : pool) th.join();
}

template <class In, class Out, class Load, class Store>
void softmax_rows_generic(const In* x, Out* y, int64_t rows, int64_t cols, int64_t ldx,
                          int64_t ldy, int nthreads, Load load, Store store) {
    parallel_range(rows, nthreads, [&](int64_t r0, int64_t r1) {
        std::vector<double> xin(static_cast<size_t>(cols)), yout(static_cast<size_t>(cols));
        for (int64_t r = r0; r < r1; ++r) {
            for (int64_t j = 0; j < cols; ++j) xin[j] = load(x[r * ldx + j]);
            softmax_row(xin.data(), yout.data(), cols);
            for (int64_t j = 0; j < cols; ++j) y[r * ldy + j] = store(yout[j]);
        }
    });
}

template <class In, class Out, class Load, class Store>
void layernorm_rows_generic(const In* x, Out* y, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t ldy, const In* gamma, const In* beta, double eps, bool gelu,
                            int nthreads, Load load, Store store) {
    std::vector<double> g, b;
    if (gamma != nullptr) {
        g.resize(static_cast<size_t>(cols));
        for (int64_t j = 0; j < cols; ++j) g[j] = load(gamma[j]);
    }
    if (beta != nullptr) {
        b.resize(static_cast<size_t>(cols));
        for (int64_t j = 0; j < cols; ++j) b[j] = load(beta[j]);
    }
    const double* gp = gamma != nullptr ? g.data() : nullptr;
    const double* bp = beta != nullptr ? b.data() : nullptr;
    parallel_range(rows, nthreads, [&](int64_t r0, int64_t r1) {
        std::vector<double> xin(static_cast<size_t>(cols)), yout(static_cast<size_t>(cols));
        for (int64_t r = r0; r < r1; ++r) {
            for (int64_t j = 0; j < cols; ++j) xin[j] = load(x[r * ldx + j]);
            layernorm_row(xin.data(), yout.data(), cols, gp, bp, eps, gelu);
            for (int64_t j = 0; j < cols; ++j) y[r * ldy + j] = store(yout[j]);
        }
    });
}

template <class T, class Load, class Store>
void softmax_bwd_rows_generic(const T* y, const T* dy, T* dx, int64_t rows, int64_t cols,
                              int nthreads, Load load, Store store) {
    parallel_range(rows, nthreads, [&](int64_t r0, int64_t r1) {
        std::vector<double> a(static_cast<size_t>(cols)), b(static_cast<size_t>(cols)),
            o(static_cast<size_t>(cols));
        for (int64_t r = r0; r < r1; ++r) {
            for (int64_t j = 0; j < cols; ++j) {
                a[j] = load(y[r * cols + j]);
                b[j] = load(dy[r * cols + j]);
            }
            softmax_bwd_row(a.data(), b.data(), o.data(), cols);
            for (int64_t j = 0; j < cols; ++j) dx[r * cols + j] = store(o[j]);
        }
    });
}

bool softmax_args_ok(const void* x, const void* y, int64_t rows, int64_t cols, int64_t ldx,
                     int64_t ldy) {
    if (rows < 0 || cols < 0) return false;
    if (rows == 0 || cols == 0) return true;
    return x != nullptr && y != nullptr && ldx >= cols && ldy >= cols;
}

}  // namespace

extern "C" {

// ---- rounding helpers (pinned against torch's own bf16 conversion) ----
void oracle_f32_to_bf16(const float* x, uint16_t* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = f32_to_bf16(x[i]);
}
void oracle_bf16_to_f32(const uint16_t* x, float* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = bf16_to_f32(x[i]);
}

// ---- GELU ----
// Unrounded real function in double (both forms), for the pins.
void oracle_gelu_tanh_f64(const double* x, double* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = gelu_real(x[i]);
}
void oracle_gelu_tanh_literal_f64(const double* x, double* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = gelu_literal(x[i]);
}
// fp32 in, fp32 out: the double result rounded once to fp32.
void oracle_gelu_tanh_f32(const float* x, float* y, int64_t n, int nthreads) {
    parallel_range(n, nthreads, [&](int64_t b, int64_t e) {
        for (int64_t i = b; i < e; ++i) y[i] = static_cast<float>(gelu_real(x[i]));
    });
}
// bf16 in, bf16 out: the fp32 result rounded to bf16.
void oracle_gelu_tanh_bf16(const uint16_t* x, uint16_t* y, int64_t n, int nthreads) {
    parallel_range(n, nthreads, [&](int64_t b, int64_t e) {
        for (int64_t i = b; i < e; ++i)
            y[i] = f32_to_bf16(static_cast<float>(gelu_real(bf16_to_f32(x[i]))));
    });
}

// ---- chain (returns 0, or -1 for an invalid op list) ----
int oracle_chain_f32(const float* x, float* y, int64_t n, const int32_t* kinds,
                     const float* scalars, int n_ops, int nthreads) {
    if (!ops_valid(kinds, n_ops)) return -1;
    parallel_range(n, nthreads, [&](int64_t b, int64_t e) {
        for (int64_t i = b; i < e; ++i) y[i] = chain_one(x[i], kinds, scalars, n_ops);
    });
    return 0;
}
int oracle_chain_bf16(const uint16_t* x, uint16_t* y, int64_t n, const int32_t* kinds,
                      const float* scalars, int n_ops, int nthreads) {
    if (!ops_valid(kinds, n_ops)) return -1;
    parallel_range(n, nthreads, [&](int64_t b, int64_t e) {
        for (int64_t i = b; i < e; ++i)
            y[i] = f32_to_bf16(chain_one(bf16_to_f32(x[i]), kinds, scalars, n_ops));
    });
    return 0;
}

// ---- row softmax (returns 0, or -1 for invalid sizes) ----
// Strides ldx, ldy are in elements; entries past cols in a row are neither
// read nor written.
int oracle_softmax_rows_f64(const double* x, double* y, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t ldy) {
    if (!softmax_args_ok(x, y, rows, cols, ldx, ldy)) return -1;
    softmax_rows_generic(x, y, rows, cols, ldx, ldy, 1, [](double v) { return v; },
                         [](double v) { return v; });
    return 0;
}
int oracle_softmax_rows_f32(const float* x, float* y, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t ldy, int nthreads) {
    if (!softmax_args_ok(x, y, rows, cols, ldx, ldy)) return -1;
    softmax_rows_generic(x, y, rows, cols, ldx, ldy, nthreads,
                         [](float v) { return static_cast<double>(v); },
                         [](double v) { return static_cast<float>(v); });
    return 0;
}
int oracle_softmax_rows_bf16(const uint16_t* x, uint16_t* y, int64_t rows, int64_t cols,
                             int64_t ldx, int64_t ldy, int nthreads) {
    if (!softmax_args_ok(x, y, rows, cols, ldx, ldy)) return -1;
    softmax_rows_generic(x, y, rows, cols, ldx, ldy, nthreads,
                         [](uint16_t v) { return static_cast<double>(bf16_to_f32(v)); },
                         [](double v) { return f32_to_bf16(static_cast<float>(v)); });
    return 0;
}

// ---- backward ----
// GELU'(x) in double, unrounded (for the pins).
void oracle_gelu_tanh_grad_f64(const double* x, double* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = gelu_grad_real(x[i]);
}
// dx = dy * GELU'(x), computed in double and rounded once.
void oracle_gelu_tanh_bwd_f32(const float* x, const float* dy, float* dx, int64_t n,
                              int nthreads) {
    parallel_range(n, nthreads, [&](int64_t b, int64_t e) {
        for (int64_t i = b; i < e; ++i)
            dx[i] = static_cast<float>(static_cast<double>(dy[i]) * gelu_grad_real(x[i]));
    });
}
void oracle_gelu_tanh_bwd_bf16(const uint16_t* x, const uint16_t* dy, uint16_t* dx, int64_t n,
                               int nthreads) {
    parallel_range(n, nthreads, [&](int64_t b, int64_t e) {
        for (int64_t i = b; i < e; ++i) {
            const double g = gelu_grad_real(bf16_to_f32(x[i]));
            dx[i] = f32_to_bf16(static_cast<float>(static_cast<double>(bf16_to_f32(dy[i])) * g));
        }
    });
}
// Softmax backward over contiguous rows (returns 0, or -1 for invalid sizes).
int oracle_softmax_bwd_rows_f64(const double* y, const double* dy, double* dx, int64_t rows,
                                int64_t cols) {
    if (rows < 0 || cols < 0 || ((rows > 0 && cols > 0) && (!y || !dy || !dx))) return -1;
    softmax_bwd_rows_generic(y, dy, dx, rows, cols, 1, [](double v) { return v; },
                             [](double v) { return v; });
    return 0;
}
int oracle_softmax_bwd_rows_f32(const float* y, const float* dy, float* dx, int64_t rows,
                                int64_t cols, int nthreads) {
    if (rows < 0 || cols < 0 || ((rows > 0 && cols > 0) && (!y || !dy || !dx))) return -1;
    softmax_bwd_rows_generic(y, dy, dx, rows, cols, nthreads,
                             [](float v) { return static_cast<double>(v); },
                             [](double v) { return static_cast<float>(v); });
    return 0;
}
int oracle_softmax_bwd_rows_bf16(const uint16_t* y, const uint16_t* dy, uint16_t* dx,
                                 int64_t rows, int64_t cols, int nthreads) {
    if (rows < 0 || cols < 0 || ((rows > 0 && cols > 0) && (!y || !dy || !dx))) return -1;
    softmax_bwd_rows_generic(y, dy, dx, rows, cols, nthreads,
                             [](uint16_t v) { return static_cast<double>(bf16_to_f32(v)); },
                             [](double v) { return f32_to_bf16(static_cast<float>(v)); });
    return 0;
}

// ---- layernorm (returns 0, or -1 for invalid sizes) ----
// gamma, beta: per-column arrays in the storage type of x, or NULL.
int oracle_layernorm_rows_f64(const double* x, double* y, int64_t rows, int64_t cols,
                              int64_t ldx, int64_t ldy, const double* gamma, const double* beta,
                              double eps, int gelu) {
    if (!softmax_args_ok(x, y, rows, cols, ldx, ldy) || !(eps >= 0.0)) return -1;
    layernorm_rows_generic(x, y, rows, cols, ldx, ldy, gamma, beta, eps, gelu != 0, 1,
                           [](double v) { return v; }, [](double v) { return v; });
    return 0;
}
int oracle_layernorm_rows_f32(const float* x, float* y, int64_t rows, int64_t cols, int64_t ldx,
                              int64_t ldy, const float* gamma, const float* beta, double eps,
                              int gelu, int nthreads) {
    if (!softmax_args_ok(x, y, rows, cols, ldx, ldy) || !(eps >= 0.0)) return -1;
    layernorm_rows_generic(x, y, rows, cols, ldx, ldy, gamma, beta, eps, gelu != 0, nthreads,
                           [](float v) { return static_cast<double>(v); },
                           [](double v) { return static_cast<float>(v); });
    return 0;
}
int oracle_layernorm_rows_bf16(const uint16_t* x, uint16_t* y, int64_t rows, int64_t cols,
                               int64_t ldx, int64_t ldy, const uint16_t* gamma,
                               const uint16_t* beta, double eps, int gelu, int nthreads) {
    if (!softmax_args_ok(x, y, rows, cols, ldx, ldy) || !(eps >= 0.0)) return -1;
    layernorm_rows_generic(x, y, rows, cols, ldx, ldy, gamma, beta, eps, gelu != 0, nthreads,
                           [](uint16_t v) { return static_cast<double>(bf16_to_f32(v)); },
                           [](double v) { return f32_to_bf16(static_cast<float>(v)); });
    return 0;
}

}  // extern "C"
