// softmax.hip -- launchers of the row softmax kernels in softmax_kernels.hpp:
// the single-pass kernel for rows up to the on-chip capacity, the online
// two-pass kernel above it.
#include <atomic>

#include <utility>

#include "launch.hpp"
#include "softmax_kernels.hpp"

namespace fk {
namespace {

// grid * block stays below 2^31 work-items (the dispatch packet holds the
// grid size in work-items as 32 bits); rows beyond it are grid-strided.
constexpr int64_t kMaxWorkItems = int64_t(1) << 31;

// ----------------------------------------------------------------- launch -
template <class... Args>
hipError_t launch_kernel(const void* fn, int64_t grid, int block, hipStream_t s, Args... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(block), argv, 0, s);
}

int64_t clamp_grid(int64_t g, int threads) {
    const int64_t cap = kMaxWorkItems / threads;
    return g < 1 ? 1 : (g > cap ? cap : g);
}

// Single-pass shapes (waves per row, 16-byte vectors per lane), smallest
// capacity first; the first that covers the row is used. At most 4 vectors
// per lane until the widest shape: on MI355X a bf16 4096-column row ran 12 %
// faster as 2 waves x 4 vectors than as 1 wave x 8 (fewer VGPRs, more waves
// in flight). The 3-, 5-, 6- and 12-wave shapes fit common model widths
// exactly (bf16 3072, 5120, 6144, 10240, 12288, 24576; fp32 1536, 2560,
// 3072, 5120, 6144, 12288): lanes left idle by a wider shape cost bandwidth
// in proportion, a row's time being set by latency.
struct RegShape {
    int wpr, vpl;
};
constexpr RegShape kRegShapes[] = {{1, 1}, {1, 2}, {1, 4},  {3, 2},  {2, 4},  {5, 2},  {3, 4},
                                   {4, 4}, {5, 4}, {6, 4},  {8, 4},  {12, 4}, {16, 4}, {16, 8}};
// Row data is read once and written once: non-temporal loads and stores
// (measured 4-9 % faster on the C4 and C5a shapes).
constexpr bool kRowNT = true;
constexpr int kNumRegShapes = sizeof(kRegShapes) / sizeof(kRegShapes[0]);

template <class IO>
constexpr int64_t reg_capacity(RegShape sh) {
    return int64_t(sh.wpr) * kWave * sh.vpl * IO::kVec;
}

template <class IO, int WPR, int VPL>
hipError_t launch_reg(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                      int64_t ldy, bool vec, hipStream_t s) {
    constexpr int kThreads = reg_threads<WPR>();
    constexpr int kRowsPerWg = kThreads / (WPR * kWave);
    const int64_t grid = clamp_grid((rows + kRowsPerWg - 1) / kRowsPerWg, kThreads);
    // a row that fills the shape exactly runs the variant without masks; a
    // width that is a multiple of the vector, the one with per-vector masks
    const void* fn =
        !vec ? reinterpret_cast<const void*>(&softmax_reg_kernel<IO, WPR, VPL, false>)
        : cols == reg_capacity<IO>(RegShape{WPR, VPL})
            ? reinterpret_cast<const void*>(&softmax_reg_kernel<IO, WPR, VPL, true, kRowNT, kFitFull>)
        : cols % IO::kVec == 0
            ? reinterpret_cast<const void*>(&softmax_reg_kernel<IO, WPR, VPL, true, kRowNT, kFitVec>)
            : reinterpret_cast<const void*>(&softmax_reg_kernel<IO, WPR, VPL, true, kRowNT>);
    return launch_kernel(fn, grid, kThreads, s, x, y, rows, cols, ldx, ldy);
}

template <class IO, size_t... I>
hipError_t dispatch_reg_i(int shape, const void* x, void* y, int64_t rows, int64_t cols,
                          int64_t ldx, int64_t ldy, bool vec, hipStream_t s,
                          std::index_sequence<I...>) {
    hipError_t r = hipErrorInvalidValue;
    ((shape == static_cast<int>(I)
          ? (r = launch_reg<IO, kRegShapes[I].wpr, kRegShapes[I].vpl>(x, y, rows, cols, ldx, ldy,
                                                                     vec, s))
          : r),
     ...);
    return r;
}

template <class IO>
hipError_t dispatch_reg(int shape, const void* x, void* y, int64_t rows, int64_t cols,
                        int64_t ldx, int64_t ldy, bool vec, hipStream_t s) {
    return dispatch_reg_i<IO>(shape, x, y, rows, cols, ldx, ldy, vec, s,
                              std::make_index_sequence<kNumRegShapes>{});
}

// Online shape: 1024 lanes per row, 16 values per lane per chunk.
constexpr int kOnlineThreads = 1024;
template <class IO>
constexpr int kOnlineVpl = IO::kVec == 4 ? 4 : 2;

template <class IO>
hipError_t launch_online(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                         int64_t ldy, bool vec, hipStream_t s) {
    constexpr int VPL = kOnlineVpl<IO>;
    const void* fn =
        vec ? reinterpret_cast<const void*>(&softmax_online_kernel<IO, kOnlineThreads, VPL, true>)
            : reinterpret_cast<const void*>(&softmax_online_kernel<IO, kOnlineThreads, VPL, false>);
    return launch_kernel(fn, clamp_grid(rows, kOnlineThreads), kOnlineThreads, s, x, y, rows, cols,
                         ldx, ldy);
}

// Split shape: 256-lane blocks, 32 values per lane -> 8192-column slices.
constexpr int kSplitThreads = 256;
template <class IO>
constexpr int kSplitVpl = 32 / IO::kVec;
template <class IO>
constexpr int64_t kSplitWidth = int64_t(kSplitThreads) * 32;

std::atomic<int64_t> g_split_wait_limit{int64_t(1) << 20};

template <class IO>
int64_t split_parts(int64_t rows, int64_t cols) {
    const int64_t parts = (cols + kSplitWidth<IO> - 1) / kSplitWidth<IO>;
    if (cols <= reg_capacity<IO>(kRegShapes[kNumRegShapes - 1])) return 0;  // on-chip path
    if (parts > kSplitMaxParts) return 0;
    if (rows > (kMaxWorkItems / kSplitThreads) / parts) return 0;  // one block per slice
    return parts;
}

int64_t split_ws_bytes(int64_t rows, int64_t parts) {
    const int64_t depart = (rows * 4 + 7) / 8 * 8;
    return rows * parts * 8 + depart;
}

template <class IO>
hipError_t launch_split(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                        int64_t ldy, int64_t parts, void* ws, bool vec, hipStream_t s) {
    constexpr int VPL = kSplitVpl<IO>;
    const void* fn =
        vec ? reinterpret_cast<const void*>(&softmax_split_kernel<IO, kSplitThreads, VPL, true, kRowNT>)
            : reinterpret_cast<const void*>(&softmax_split_kernel<IO, kSplitThreads, VPL, false>);
    auto* slots = static_cast<unsigned long long*>(ws);
    auto* depart = reinterpret_cast<unsigned int*>(slots + rows * parts);
    const int p = static_cast<int>(parts);
    const int64_t spin = g_split_wait_limit.load(std::memory_order_relaxed);
    return launch_kernel(fn, rows * parts, kSplitThreads, s, x, y, rows, cols, ldx, ldy, p, slots,
                         depart, spin);
}

__global__ __launch_bounds__(256) void zero_fill_kernel(unsigned long long* p, int64_t n) {
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) p[i] = 0ull;
}

template <class IO>
hipError_t launch_softmax_t(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t ldy, bool online, void* ws, int64_t ws_bytes, hipStream_t s) {
    const bool vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0 &&
                     (ldx * IO::kBytes) % 16 == 0 && (ldy * IO::kBytes) % 16 == 0;
    if (!online) {
        for (int i = 0; i < kNumRegShapes; ++i)
            if (cols <= reg_capacity<IO>(kRegShapes[i]))
                return dispatch_reg<IO>(i, x, y, rows, cols, ldx, ldy, vec, s);
        const int64_t parts = split_parts<IO>(rows, cols);
        if (parts > 0 && ws != nullptr && ws_bytes >= split_ws_bytes(rows, parts))
            return launch_split<IO>(x, y, rows, cols, ldx, ldy, parts, ws, vec, s);
    }
    return launch_online<IO>(x, y, rows, cols, ldx, ldy, vec, s);
}

}  // namespace

int64_t softmax_onchip_max_cols(Dtype dt) {
    return dt == kF32 ? reg_capacity<IoF32>(kRegShapes[kNumRegShapes - 1])
                      : reg_capacity<IoBF16>(kRegShapes[kNumRegShapes - 1]);
}

int64_t softmax_workspace_bytes(int64_t rows, int64_t cols, Dtype dt) {
    const int64_t parts = dt == kF32 ? split_parts<IoF32>(rows, cols) : split_parts<IoBF16>(rows, cols);
    return parts > 0 ? split_ws_bytes(rows, parts) : 0;
}

int64_t split_wait_limit() { return g_split_wait_limit.load(); }

int64_t set_split_wait_limit(int64_t polls) { return g_split_wait_limit.exchange(polls); }

hipError_t launch_zero_fill(void* p, int64_t nbytes, hipStream_t s) {
    const int64_t n = nbytes / 8;
    const int64_t grid = n / 256 + 1 < 4096 ? n / 256 + 1 : 4096;
    return launch_kernel(reinterpret_cast<const void*>(&zero_fill_kernel), grid, 256, s,
                         static_cast<unsigned long long*>(p), n);
}

hipError_t launch_softmax(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                          int64_t ldy, Dtype dt, bool online, void* ws, int64_t ws_bytes,
                          hipStream_t s) {
    return dt == kF32 ? launch_softmax_t<IoF32>(x, y, rows, cols, ldx, ldy, online, ws, ws_bytes, s)
                      : launch_softmax_t<IoBF16>(x, y, rows, cols, ldx, ldy, online, ws, ws_bytes, s);
}

}  // namespace fk
