// layernorm.hip -- launcher of the fused LayerNorm row kernel
// (layernorm_kernels.hpp). Rows up to the on-chip capacity of the row
// shapes below; wider rows are refused by the C ABI.
#include <utility>

#include "launch.hpp"
#include "layernorm_kernels.hpp"

namespace fk {
namespace {

template <class... Args>
hipError_t launch_kernel(const void* fn, int64_t grid, int block, hipStream_t s, Args... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(block), argv, 0, s);
}

// Row shapes (waves per row, 16-byte vectors per lane), smallest capacity
// first; the first that covers the row is used. At most 2 vectors per lane
// until the widest shapes: a lane also holds gamma and beta of its columns,
// so the LayerNorm needs about three registers per value where the softmax
// needs one (bf16 4096 columns: 4 waves x 2 vectors, 80 VGPRs, 6 waves per
// SIMD). Besides the powers of two, 3, 5, 6, 10 and 12 waves fit common
// model widths exactly (bf16 1536, 2560, 3072, 5120, 6144, 12288; fp32 768,
// 1536, 2560, 3072, 5120, 6144): a row time is set by latency, so lanes
// left idle by a wider shape cost bandwidth in proportion.
struct LnShape {
    int wpr, vpl;
};
constexpr LnShape kLnShapes[] = {{1, 1},  {1, 2},  {3, 1},  {2, 2},  {5, 1},  {3, 2},
                                 {4, 2},  {5, 2},  {6, 2},  {8, 2},  {10, 2}, {12, 2},
                                 {16, 2}, {12, 4}, {16, 4}, {16, 8}};
constexpr int kNumLnShapes = sizeof(kLnShapes) / sizeof(kLnShapes[0]);
constexpr bool kLnNT = true;  // x read once, y written once

template <class IO>
constexpr int64_t ln_capacity(LnShape sh) {
    return int64_t(sh.wpr) * kWave * sh.vpl * IO::kVec;
}

// the per-vector-mask variant exists for the shapes that hold gamma and beta
// (kFitAny elsewhere, so no unused kernel is compiled)
template <int VPL>
constexpr int ln_vfit() {
    return VPL <= kLnHoldAffineVpl ? kFitVec : kFitAny;
}

// Workgroups of one launch at most: a workgroup loads gamma and beta once
// and then strides over rows, so capping the grid cuts the gamma/beta reads
// (16 KiB per workgroup on a 4096-column bf16 row) from one per row to one
// per workgroup. On MI355X, bf16 32768 x 4096 with GELU: 102 us with a
// workgroup per row, 93 us at 8192 workgroups, 92 us at 16384.
constexpr int64_t kLnMaxGrid = 16384;

template <class IO, int WPR, int VPL>
hipError_t launch_ln(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy,
                     const void* g, const void* b, float eps, int gelu, bool vec, hipStream_t s) {
    constexpr int kThreads = reg_threads<WPR>();
    constexpr int kRowsPerWg = kThreads / (WPR * kWave);
    int64_t grid = (rows + kRowsPerWg - 1) / kRowsPerWg;
    if (grid > kLnMaxGrid) grid = kLnMaxGrid;
    // a row that fills the shape exactly runs the variant without masks; a
    // width that is a multiple of the vector, the one with per-vector masks
    // (on the shapes that hold gamma and beta: on the widest ones that
    // variant needs far more registers than the 128 a 1024-lane workgroup
    // allows, and spills)
    const int fit = !vec ? kFitAny
                    : cols == ln_capacity<IO>(LnShape{WPR, VPL}) ? kFitFull
                    : (cols % IO::kVec == 0 && VPL <= kLnHoldAffineVpl) ? kFitVec
                                                                        : kFitAny;
    const void* fn = nullptr;
    if (!vec)
        fn = gelu ? reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, false, true>)
                  : reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, false, false>);
    else if (fit == kFitFull)
        fn = gelu ? reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, true, true, kLnNT, kFitFull>)
                  : reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, true, false, kLnNT, kFitFull>);
    else if (VPL <= kLnHoldAffineVpl && fit == kFitVec)
        fn = gelu ? reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, true, true, kLnNT, ln_vfit<VPL>()>)
                  : reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, true, false, kLnNT, ln_vfit<VPL>()>);
    else
        fn = gelu ? reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, true, true, kLnNT>)
                  : reinterpret_cast<const void*>(&layernorm_reg_kernel<IO, WPR, VPL, true, false, kLnNT>);
    return launch_kernel(fn, grid, kThreads, s, x, y, rows, cols, ldx, ldy, g, b, eps);
}

// launch_ln for shape index `shape` of kLnShapes
template <class IO, size_t... I>
hipError_t dispatch_ln(int shape, const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                       int64_t ldy, const void* g, const void* b, float eps, int gelu, bool vec,
                       hipStream_t s, std::index_sequence<I...>) {
    hipError_t r = hipErrorInvalidValue;
    ((shape == static_cast<int>(I)
          ? (r = launch_ln<IO, kLnShapes[I].wpr, kLnShapes[I].vpl>(x, y, rows, cols, ldx, ldy, g,
                                                                  b, eps, gelu, vec, s))
          : r),
     ...);
    return r;
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
    return dispatch_ln<IO>(shape, x, y, rows, cols, ldx, ldy, g, b, eps, gelu, vec, s,
                           std::make_index_sequence<kNumLnShapes>{});
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
