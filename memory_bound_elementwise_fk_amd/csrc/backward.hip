// backward.hip -- launchers of the backward kernels (backward_kernels.hpp):
// GELU backward (elementwise, two inputs) and row softmax backward.
#include "backward_kernels.hpp"
#include <utility>

#include "launch.hpp"

namespace fk {
namespace {

constexpr int64_t kMaxWorkItems = int64_t(1) << 31;

template <class... Args>
hipError_t launch_kernel(const void* fn, int64_t grid, int block, hipStream_t s, Args... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(block), argv, 0, s);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// One 16-byte vector per lane and operand, non-temporal (every operand is
// read or written once), the forward GELU's workgroup sizes.
template <class IO>
constexpr int kBwdT = IO::kBytes == 2 ? 128 : 64;

template <class IO, class Op>
hipError_t launch_ew2(const void* a, const void* b, void* out, int64_t n, const Op& op,
                      hipStream_t s) {
    if (aligned16(a) && aligned16(b) && aligned16(out)) {
        constexpr int T = kBwdT<IO>;
        const int64_t nfull = (n / IO::kVec) / T;
        const int64_t ntiles = (n + int64_t(T) * IO::kVec - 1) / (int64_t(T) * IO::kVec);
        const auto* av = static_cast<const u32x4*>(a);
        const auto* bv = static_cast<const u32x4*>(b);
        auto* ov = static_cast<u32x4*>(out);
        if (ntiles <= kMaxWorkItems / T)
            return launch_kernel(reinterpret_cast<const void*>(&ew2_vec_kernel<IO, T, true, false, Op>),
                                 ntiles, T, s, av, bv, ov, n, nfull, op);
        return launch_kernel(reinterpret_cast<const void*>(&ew2_vec_kernel<IO, T, true, true, Op>),
                             kMaxWorkItems / T, T, s, av, bv, ov, n, nfull, op);
    }
    constexpr int T = 256, PER = 8;
    int64_t grid = (n + int64_t(T) * PER - 1) / (int64_t(T) * PER);
    if (grid > kMaxWorkItems / T) grid = kMaxWorkItems / T;
    return launch_kernel(reinterpret_cast<const void*>(&ew2_scalar_kernel<IO, T, PER, Op>), grid, T,
                         s, a, b, out, n, op);
}

// Softmax backward row shapes: as the forward table without its widest
// entry (two operands per lane are held in registers).
struct BwdShape {
    int wpr, vpl;
};
constexpr BwdShape kBwdShapes[] = {{1, 1}, {1, 2}, {1, 4}, {3, 2}, {2, 4},  {5, 2}, {3, 4},
                                   {4, 4}, {5, 4}, {6, 4}, {8, 4}, {12, 4}, {16, 4}};
constexpr int kNumBwdShapes = sizeof(kBwdShapes) / sizeof(kBwdShapes[0]);

template <class IO>
constexpr int64_t bwd_capacity(BwdShape sh) {
    return int64_t(sh.wpr) * kWave * sh.vpl * IO::kVec;
}

template <class IO, int WPR, int VPL>
hipError_t launch_sbwd(const void* y, const void* dy, void* dx, int64_t rows, int64_t cols,
                       int64_t ldy, int64_t lddy, int64_t lddx, bool vec, hipStream_t s) {
    constexpr int kThreads = reg_threads<WPR>();
    constexpr int kRowsPerWg = kThreads / (WPR * kWave);
    int64_t grid = (rows + kRowsPerWg - 1) / kRowsPerWg;
    if (grid > kMaxWorkItems / kThreads) grid = kMaxWorkItems / kThreads;
    // a row that fills the shape exactly runs the variant without masks; a
    // width that is a multiple of the vector, the one with per-vector masks
    const void* fn =
        !vec ? reinterpret_cast<const void*>(&softmax_bwd_reg_kernel<IO, WPR, VPL, false>)
        : cols == bwd_capacity<IO>(BwdShape{WPR, VPL})
            ? reinterpret_cast<const void*>(&softmax_bwd_reg_kernel<IO, WPR, VPL, true, true, kFitFull>)
        : cols % IO::kVec == 0
            ? reinterpret_cast<const void*>(&softmax_bwd_reg_kernel<IO, WPR, VPL, true, true, kFitVec>)
            : reinterpret_cast<const void*>(&softmax_bwd_reg_kernel<IO, WPR, VPL, true, true>);
    return launch_kernel(fn, grid, kThreads, s, y, dy, dx, rows, cols, ldy, lddy, lddx);
}

template <class IO, size_t... I>
hipError_t dispatch_sbwd(int shape, const void* y, const void* dy, void* dx, int64_t rows,
                         int64_t cols, int64_t ldy, int64_t lddy, int64_t lddx, bool vec,
                         hipStream_t s, std::index_sequence<I...>) {
    hipError_t r = hipErrorInvalidValue;
    ((shape == static_cast<int>(I)
          ? (r = launch_sbwd<IO, kBwdShapes[I].wpr, kBwdShapes[I].vpl>(y, dy, dx, rows, cols, ldy,
                                                                      lddy, lddx, vec, s))
          : r),
     ...);
    return r;
}

template <class IO>
hipError_t launch_sbwd_t(const void* y, const void* dy, void* dx, int64_t rows, int64_t cols,
                         int64_t ldy, int64_t lddy, int64_t lddx, hipStream_t s) {
    const uintptr_t addr = reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(dy) |
                           reinterpret_cast<uintptr_t>(dx);
    const bool vec = (addr & 15u) == 0 && (ldy * IO::kBytes) % 16 == 0 &&
                     (lddy * IO::kBytes) % 16 == 0 && (lddx * IO::kBytes) % 16 == 0;
    int shape = 0;
    while (shape < kNumBwdShapes - 1 && cols > bwd_capacity<IO>(kBwdShapes[shape])) ++shape;
    return dispatch_sbwd<IO>(shape, y, dy, dx, rows, cols, ldy, lddy, lddx, vec, s,
                             std::make_index_sequence<kNumBwdShapes>{});
}

}  // namespace

hipError_t launch_gelu_backward(const void* x, const void* dy, void* dx, int64_t n, Dtype dt,
                                hipStream_t s) {
    return dt == kF32 ? launch_ew2<IoF32>(x, dy, dx, n, GeluBwdOp{}, s)
                      : launch_ew2<IoBF16>(x, dy, dx, n, GeluBwdOp{}, s);
}

int64_t softmax_backward_max_cols(Dtype dt) {
    return dt == kF32 ? bwd_capacity<IoF32>(kBwdShapes[kNumBwdShapes - 1])
                      : bwd_capacity<IoBF16>(kBwdShapes[kNumBwdShapes - 1]);
}

hipError_t launch_softmax_backward(const void* y, const void* dy, void* dx, int64_t rows,
                                   int64_t cols, int64_t ldy, int64_t lddy, int64_t lddx,
                                   Dtype dt, hipStream_t s) {
    return dt == kF32 ? launch_sbwd_t<IoF32>(y, dy, dx, rows, cols, ldy, lddy, lddx, s)
                      : launch_sbwd_t<IoBF16>(y, dy, dx, rows, cols, ldy, lddy, lddx, s);
}

}  // namespace fk
