// layernorm.hip -- launcher of the fused LayerNorm row kernel
// (layernorm_kernels.hpp). Rows up to the on-chip capacity of the row
// shapes below; wider rows are refused by the C ABI.
#include "launch.hpp"
#include "layernorm_kernels.hpp"

namespace fk {
namespace {

constexpr int64_t kMaxWorkItems = int64_t(1) << 31;

template <class... Args>
hipError_t launch_kernel(const void* fn, int64_t grid, int block, hipStream_t s, Args... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(block), argv, 0, s);
}

// Row shapes (waves per row, 16-byte vectors per lane), smallest first; the
// first that covers the row is used. At most 2 vectors per lane until the
// widest shapes: a lane also holds gamma and beta of its columns, so the
// LayerNorm needs about three registers per value where the softmax needs
// one (bf16 4096 columns: 4 waves x 2 vectors, 83 VGPRs, 5 waves per SIMD).
struct LnShape {
    int wpr, vpl;
};
constexpr LnShape kLnShapes[] = {{1, 1}, {1, 2}, {2, 2}, {4, 2}, {8, 2}, {16, 2}, {16, 4}, {16, 8}};
constexpr int kNumLnShapes = sizeof(kLnShapes) / sizeof(kLnShapes[0]);
constexpr bool kLnNT = true;  // x read once, y written once

template <class IO>
constexpr int64_t ln_capacity(LnShape sh) {
    return int64_t(sh.wpr) * kWave * sh.vpl * IO::kVec;
}

template <class IO, int WPR, int VPL>
hipError_t launch_ln(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy,
                     const void* g, const void* b, float eps, int gelu, bool vec, hipStream_t s) {
    constexpr int kThreads = reg_threads<WPR>();
    constexpr int kRowsPerWg = kThreads / (WPR * kWave);
    int64_t grid = (rows + kRowsPerWg - 1) / kRowsPerWg;
    if (grid > kMaxWorkItems / kThreads) grid = kMaxWorkItems / kThreads;
    // a row that fills the shape exactly runs the variant without masks
    const bool full = vec && cols == ln_capacity<IO>(LnShape{WPR, VPL});
    const void* fn =
        full ? (gelu ? reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, true, true, kLnNT, true>)
                     : reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, true, false, kLnNT, true>))
        : vec ? (gelu ? reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, true, true, kLnNT>)
                      : reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, true, false, kLnNT>))
              : (gelu ? reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, false, true>)
                      : reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, false, false>));
    return launch_kernel(fn, grid, kThreads, s, x, y, rows, cols, ldx, ldy, g, b, eps);
}

template <class IO>
hipError_t launch_ln_t(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                       int64_t ldy, const void* g, const void* b, float eps, int gelu,
                       hipStream_t s) {
    const uintptr_t addr = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y) |
                           reinterpret_cast<uintptr_t>(g) | reinterpret_cast<uintptr_t>(b);
    const bool vec = (addr & 15u) == 0 && (ldx * IO::kBytes) % 16 == 0 &&
                     (ldy * IO::kBytes) % 16 == 0;
    int shape = 0;
    while (shape < kNumLnShapes - 1 && cols > ln_capacity<IO>(kLnShapes[shape])) ++shape;
    switch (shape) {
        case 0: return launch_ln<IO, 1, 1>(x, y, rows, cols, ldx, ldy, g, b, eps, gelu, vec, s);
        case 1: return launch_ln<IO, 1, 2>(x, y, rows, cols, ldx, ldy, g, b, eps, gelu, vec, s);
        case 2: return launch_ln<IO, 2, 2>(x, y, rows, cols, ldx, ldy, g, b, eps, gelu, vec, s);
        case 3: return launch_ln<IO, 4, 2>(x, y, rows, cols, ldx, ldy, g, b, eps, gelu, vec, s);
        case 4: return launch_ln<IO, 8, 2>(x, y, rows, cols, ldx, ldy, g, b, eps, gelu, vec, s);
        case 5: return launch_ln<IO, 16, 2>(x, y, rows, cols, ldx, ldy, g, b, eps, gelu, vec, s);
        case 6: return launch_ln<IO, 16, 4>(x, y, rows, cols, ldx, ldy, g, b, eps, gelu, vec, s);
        default: return launch_ln<IO, 16, 8>(x, y, rows, cols, ldx, ldy, g, b, eps, gelu, vec, s);
    }
}

}  // namespace

int64_t layernorm_max_cols(Dtype dt) {
    return dt == kF32 ? ln_capacity<IoF32>(kLnShapes[kNumLnShapes - 1])
                      : ln_capacity<IoBF16>(kLnShapes[kNumLnShapes - 1]);
}

hipError_t launch_layernorm(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t ldy, const void* gamma, const void* beta, float eps, int gelu,
                            Dtype dt, hipStream_t s) {
    return dt == kF32 ? launch_ln_t<IoF32>(x, y, rows, cols, ldx, ldy, gamma, beta, eps, gelu, s)
                      : launch_ln_t<IoBF16>(x, y, rows, cols, ldx, ldy, gamma, beta, eps, gelu, s);
}

}  // namespace fk
