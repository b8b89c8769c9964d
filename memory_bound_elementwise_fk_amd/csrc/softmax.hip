// softmax.hip -- launchers of the row softmax kernels in softmax_kernels.hpp:
// the single-pass kernel for rows up to the on-chip capacity; above it the
// split kernel when the caller brings a workspace, else the online kernel.
#include <atomic>
#include <mutex>
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

// Online shape: 1024 lanes per row, 16 values per lane per chunk, for
// unaligned rows (the plain online kernel, which streams the whole row
// twice). Aligned rows run the staged kernel with 512 lanes (two waves per
// SIMD, up to 256 VGPRs per lane): 8192-column chunks, the first RREG held
// in VGPRs and the next RLDS in LDS -- 131072 fp32 or 262144 bf16 columns
// (512 KiB) of the row on chip, one workgroup per CU.
constexpr int kOnlineThreads = 1024;
template <class IO>
constexpr int kOnlineVpl = IO::kVec == 4 ? 4 : 2;
constexpr int kStagedThreads = 512;
template <class IO>
constexpr int kStagedVpl = IO::kVec == 4 ? 4 : 2;     // one 16-byte vector = 4 fp32 / 8 bf16
template <class IO>
constexpr int kStagedReg = IO::kVec == 4 ? 12 : 24;   // 192 VGPRs of raw words
template <class IO>
constexpr int kStagedLds = IO::kVec == 4 ? 4 : 8;     // 128 KiB of LDS

// The staged kernel addresses a row with 32-bit byte offsets.
constexpr int64_t kStagedMaxRowBytes = int64_t(1) << 31;

template <class IO>
hipError_t launch_online(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                         int64_t ldy, bool vec, hipStream_t s) {
    constexpr int64_t kStagedChunk = int64_t(kStagedThreads) * kStagedVpl<IO> * IO::kVec;
    // rows of exactly the chunks that stay on chip (131072 fp32 / 262144
    // bf16 columns): the rolling kernel, one workgroup per CU (its LDS allows
    // no second one), each looping over rows
    const int cus = device_cus();
    if (vec && cus > 0 && cols == (kStagedReg<IO> + kStagedLds<IO>) * kStagedChunk) {
        const void* fn = reinterpret_cast<const void*>(
            &softmax_rolling_kernel<IO, kStagedThreads, kStagedVpl<IO>, kStagedReg<IO>,
                                    kStagedLds<IO>, kRowNT>);
        return launch_kernel(fn, rows < cus ? rows : cus, kStagedThreads, s, x, y, rows, cols, ldx,
                             ldy);
    }
    if (vec && cols * IO::kBytes < kStagedMaxRowBytes) {
        const void* fn = reinterpret_cast<const void*>(
            &softmax_staged_kernel<IO, kStagedThreads, kStagedVpl<IO>, kStagedReg<IO>,
                                   kStagedLds<IO>, kRowNT>);
        return launch_kernel(fn, clamp_grid(rows, kStagedThreads), kStagedThreads, s, x, y, rows,
                             cols, ldx, ldy);
    }
    constexpr int VPL = kOnlineVpl<IO>;
    const void* fn = vec ? reinterpret_cast<const void*>(
                               &softmax_online_kernel<IO, kOnlineThreads, VPL, true>)
                         : reinterpret_cast<const void*>(
                               &softmax_online_kernel<IO, kOnlineThreads, VPL, false>);
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
// Tag of the next split launch (never 0, so a zeroed workspace holds no
// valid slot); wraps after 2^32 launches.
std::atomic<uint32_t> g_split_epoch{0};

uint32_t next_split_epoch() {
    uint32_t e = g_split_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    while (e == 0) e = g_split_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    return e;
}

template <class IO>
int64_t split_parts(int64_t rows, int64_t cols) {
    if (cols <= reg_capacity<IO>(kRegShapes[kNumRegShapes - 1])) return 0;  // on-chip path
    if (cols > kSplitMaxParts * kSplitWidth<IO>) return 0;  // more than 64 slices
    const int64_t parts = (cols + kSplitWidth<IO> - 1) / kSplitWidth<IO>;  // (no overflow now)
    if (rows > (kMaxWorkItems / kSplitThreads) / parts) return 0;  // one block per slice
    return parts;
}

// two tagged 64-bit words per slice of every row
int64_t split_ws_bytes(int64_t rows, int64_t parts) { return rows * parts * 16; }

template <class IO>
hipError_t launch_split(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                        int64_t ldy, int64_t parts, void* ws, bool vec, hipStream_t s) {
    constexpr int VPL = kSplitVpl<IO>;
    const void* fn =
        vec ? reinterpret_cast<const void*>(&softmax_split_kernel<IO, kSplitThreads, VPL, true, kRowNT>)
            : reinterpret_cast<const void*>(&softmax_split_kernel<IO, kSplitThreads, VPL, false>);
    auto* slots = static_cast<unsigned long long*>(ws);
    const int p = static_cast<int>(parts);
    const uint32_t epoch = next_split_epoch();
    const int64_t spin = g_split_wait_limit.load(std::memory_order_relaxed);
    return launch_kernel(fn, rows * parts, kSplitThreads, s, x, y, rows, cols, ldx, ldy, p, slots,
                         epoch, spin);
}

// The one place that decides the path: the launch below and the host query
// softmax_path both call it.
template <class IO>
SoftmaxPath choose_path(int64_t rows, int64_t cols, bool in_place, bool online, int64_t ws_bytes,
                        int* shape, int64_t* parts) {
    if (!online) {
        for (int i = 0; i < kNumRegShapes; ++i)
            if (cols <= reg_capacity<IO>(kRegShapes[i])) {
                *shape = i;
                return kPathOnChip;
            }
        const int64_t p = split_parts<IO>(rows, cols);
        // in place, the split path's fallback could re-read values that
        // another slice of the row has already overwritten
        if (p > 0 && !in_place && ws_bytes >= split_ws_bytes(rows, p)) {
            *parts = p;
            return kPathSplit;
        }
    }
    return kPathOnline;
}

template <class IO>
hipError_t launch_softmax_t(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t ldy, bool online, void* ws, int64_t ws_bytes, hipStream_t s) {
    const bool vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0 &&
                     (ldx * IO::kBytes) % 16 == 0 && (ldy * IO::kBytes) % 16 == 0;
    int shape = 0;
    int64_t parts = 0;
    const SoftmaxPath path =
        choose_path<IO>(rows, cols, x == y, online, ws == nullptr ? 0 : ws_bytes, &shape, &parts);
    if (path == kPathOnChip) return dispatch_reg<IO>(shape, x, y, rows, cols, ldx, ldy, vec, s);
    if (path == kPathSplit) return launch_split<IO>(x, y, rows, cols, ldx, ldy, parts, ws, vec, s);
    return launch_online<IO>(x, y, rows, cols, ldx, ldy, vec, s);
}

// The split path's slots for callers that cannot allocate: a file-scope
// device array (each GPU the library runs on holds its own copy until the
// process ends). Host code never uses the symbol itself -- on the host it is
// a stand-in, not a device address -- but the address hipGetSymbolAddress
// returns for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[kSoftmaxScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

}  // namespace

hipError_t softmax_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

int64_t softmax_onchip_max_cols(Dtype dt) {
    return dt == kF32 ? reg_capacity<IoF32>(kRegShapes[kNumRegShapes - 1])
                      : reg_capacity<IoBF16>(kRegShapes[kNumRegShapes - 1]);
}

int64_t softmax_workspace_bytes(int64_t rows, int64_t cols, Dtype dt) {
    const int64_t parts = dt == kF32 ? split_parts<IoF32>(rows, cols) : split_parts<IoBF16>(rows, cols);
    return parts > 0 ? split_ws_bytes(rows, parts) : 0;
}

SoftmaxPath softmax_path(int64_t rows, int64_t cols, Dtype dt, bool in_place, bool online,
                         int64_t ws_bytes) {
    int shape = 0;
    int64_t parts = 0;
    return dt == kF32 ? choose_path<IoF32>(rows, cols, in_place, online, ws_bytes, &shape, &parts)
                      : choose_path<IoBF16>(rows, cols, in_place, online, ws_bytes, &shape, &parts);
}

int64_t split_wait_limit() { return g_split_wait_limit.load(); }

int64_t set_split_wait_limit(int64_t polls) { return g_split_wait_limit.exchange(polls); }

hipError_t launch_softmax(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                          int64_t ldy, Dtype dt, bool online, void* ws, int64_t ws_bytes,
                          hipStream_t s) {
    return dt == kF32 ? launch_softmax_t<IoF32>(x, y, rows, cols, ldx, ldy, online, ws, ws_bytes, s)
                      : launch_softmax_t<IoBF16>(x, y, rows, cols, ldx, ldy, online, ws, ws_bytes, s);
}

}  // namespace fk
