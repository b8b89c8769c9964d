// softmax.hip -- row softmax kernels for gfx950.
//
// The operation, per row: m = max_j x_j; s = sum_j exp(x_j - m);
// y_j = exp(x_j - m) / s ("CS336 lecture 6" notes, section 5.2: one block
// per row, load the row on chip, max, exponentials and sum, normalise,
// write back). exp(x - m) is evaluated as 2^((x - m) log2e) with the
// hardware exp2; the max element gives exactly 2^0 = 1, so a one-column row
// is exactly 1 and a constant row of 2^k columns exactly 2^-k.
//
// Single-pass kernel (rows up to the on-chip capacity): the row is held in
// the VGPRs of the lanes that own it -- WPR waves per row, VPL 16-byte
// vectors per lane -- so HBM is read once and written once. Reductions run
// lane-local, then across the wave with DPP moves, then across the row's
// waves through LDS, always in a fixed order (bitwise reproducible).
//
// Online kernel (any width, used above the capacity): one workgroup per row
// streams the row in chunks keeping a per-lane running max m and running
// sum l; when the max grows, l is rescaled by 2^((m_old - m_new) log2e)
// ("Lecture 6: GPU Kernels and Triton", section 7.2 "Online Softmax", here
// without the attention accumulator). Lane states merge by the same rule.
// Pass 2 re-reads the row, last chunk first (the most recently read bytes
// are the likeliest to still be in L2 / Infinity Cache), and writes
// 2^((x - m) log2e) / l.
#include "device_common.hpp"
#include "launch.hpp"

namespace fk {
namespace {

constexpr float kNegInf = -__builtin_inff();
// grid * block stays below 2^31 work-items (the dispatch packet holds the
// grid size in work-items as 32 bits); rows beyond it are grid-strided.
constexpr int64_t kMaxWorkItems = int64_t(1) << 31;

template <class IO>
__device__ inline const char* row_ptr(const void* p, int64_t row, int64_t ld) {
    return static_cast<const char*>(p) + row * ld * IO::kBytes;
}
template <class IO>
__device__ inline char* row_ptr(void* p, int64_t row, int64_t ld) {
    return static_cast<char*>(p) + row * ld * IO::kBytes;
}

// Load the E = VPL*V values a lane owns in one span of a row, starting at
// column c0. VEC layout: vectors k*LANES + lane (16-byte loads); scalar
// layout: columns k*LANES + lane. Columns >= cols read as -inf.
template <class IO, int VPL, int LANES, bool VEC>
__device__ inline void load_span(const char* xr, int64_t cols, int64_t c0, int lane,
                                 float (&v)[VPL * IO::kVec]) {
    constexpr int V = IO::kVec;
    if constexpr (VEC) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int64_t c = c0 + (int64_t(k) * LANES + lane) * V;
            if (c + V <= cols) {
                IO::unpack(ld16<false>(reinterpret_cast<const u32x4*>(xr + c * IO::kBytes)),
                           &v[k * V]);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    v[k * V + e] = (c + e < cols) ? IO::load1(xr, c + e) : kNegInf;
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < VPL * V; ++k) {
            const int64_t c = c0 + int64_t(k) * LANES + lane;
            v[k] = c < cols ? IO::load1(xr, c) : kNegInf;
        }
    }
}

template <class IO, int VPL, int LANES, bool VEC>
__device__ inline void store_span(char* yr, int64_t cols, int64_t c0, int lane,
                                  const float (&v)[VPL * IO::kVec]) {
    constexpr int V = IO::kVec;
    if constexpr (VEC) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int64_t c = c0 + (int64_t(k) * LANES + lane) * V;
            if (c + V <= cols) {
                st16<false>(reinterpret_cast<u32x4*>(yr + c * IO::kBytes), IO::pack(&v[k * V]));
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    if (c + e < cols) IO::store1(yr, c + e, v[k * V + e]);
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < VPL * V; ++k) {
            const int64_t c = c0 + int64_t(k) * LANES + lane;
            if (c < cols) IO::store1(yr, c, v[k]);
        }
    }
}

template <int WPR>
constexpr int reg_threads() {
    return WPR * kWave > 256 ? WPR * kWave : 256;
}

// ------------------------------------------------- single-pass kernel -----
template <class IO, int WPR, int VPL, bool VEC>
__global__ __launch_bounds__(reg_threads<WPR>()) void softmax_reg_kernel(
    const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy) {
    constexpr int V = IO::kVec;
    constexpr int E = VPL * V;
    constexpr int kRowLanes = WPR * kWave;
    constexpr int kRowsPerWg = reg_threads<WPR>() / kRowLanes;
    __shared__ float red[kRowsPerWg * WPR];

    const int sub = threadIdx.x / kRowLanes;  // which row of the WG
    const int lr = threadIdx.x % kRowLanes;   // lane within the row's lanes
    const int wave = lr / kWave;
    const int lane = threadIdx.x % kWave;

    // Every wave runs every iteration (the barriers are workgroup-wide);
    // a row index past the end only masks its loads and stores.
    for (int64_t rb = int64_t(blockIdx.x) * kRowsPerWg; rb < rows;
         rb += int64_t(gridDim.x) * kRowsPerWg) {
        const int64_t row = rb + sub;
        const bool active = row < rows;
        float v[E];
        if (active) {
            load_span<IO, VPL, kRowLanes, VEC>(row_ptr<IO>(x, row, ldx), cols, 0, lr, v);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i) v[i] = kNegInf;
        }

        // row max
        float m = kNegInf;
#pragma unroll
        for (int i = 0; i < E; ++i) m = fmaxf(m, v[i]);
        m = wave_max(m);
        if constexpr (WPR > 1) {
            if (lane == 0) red[sub * WPR + wave] = m;
            __syncthreads();
            m = red[sub * WPR];
#pragma unroll
            for (int w = 1; w < WPR; ++w) m = fmaxf(m, red[sub * WPR + w]);
            __syncthreads();
        }

        // exponentials and their sum (masked columns give 2^-inf = 0)
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const float e = exp2_full((v[i] - m) * kLog2e);
            v[i] = e;
            s += e;
        }
        s = wave_sum(s);
        if constexpr (WPR > 1) {
            if (lane == 0) red[sub * WPR + wave] = s;
            __syncthreads();
            s = red[sub * WPR];
#pragma unroll
            for (int w = 1; w < WPR; ++w) s += red[sub * WPR + w];
            __syncthreads();
        }

        // normalise and write back
        const float r = 1.0f / s;
#pragma unroll
        for (int i = 0; i < E; ++i) v[i] *= r;
        if (active) store_span<IO, VPL, kRowLanes, VEC>(row_ptr<IO>(y, row, ldy), cols, 0, lr, v);
    }
}

// ---------------------------------------------------------- online kernel -
template <class IO, int THREADS, int VPL, bool VEC>
__global__ __launch_bounds__(THREADS) void softmax_online_kernel(
    const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy) {
    constexpr int E = VPL * IO::kVec;
    constexpr int64_t kChunk = int64_t(THREADS) * E;
    constexpr int kWaves = THREADS / kWave;
    __shared__ float red_m[kWaves];
    __shared__ float red_l[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int64_t nchunks = (cols + kChunk - 1) / kChunk;

    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const char* xr = row_ptr<IO>(x, row, ldx);
        char* yr = row_ptr<IO>(y, row, ldy);

        // pass 1: running (m, l) per lane
        float m = kNegInf, l = 0.0f;
        for (int64_t c = 0; c < nchunks; ++c) {
            float v[E];
            load_span<IO, VPL, THREADS, VEC>(xr, cols, c * kChunk, tid, v);
            float cm = kNegInf;
#pragma unroll
            for (int i = 0; i < E; ++i) cm = fmaxf(cm, v[i]);
            const float mn = fmaxf(m, cm);
            if (mn != kNegInf) {  // while every value seen is -inf, l stays 0
                if (mn != m) l *= __builtin_amdgcn_exp2f((m - mn) * kLog2e);
                m = mn;
#pragma unroll
                for (int i = 0; i < E; ++i) l += __builtin_amdgcn_exp2f((v[i] - m) * kLog2e);
            }
        }

        // merge the lanes' states: wave (DPP), then the waves (LDS)
        wave_ml(m, l);
        if (lane == 0) {
            red_m[wave] = m;
            red_l[wave] = l;
        }
        __syncthreads();
        m = red_m[0];
        l = red_l[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) ml_merge(m, l, red_m[w], red_l[w]);
        __syncthreads();

        // pass 2: normalise, last chunk first
        const float r = 1.0f / l;
        for (int64_t c = nchunks - 1; c >= 0; --c) {
            float v[E];
            load_span<IO, VPL, THREADS, VEC>(xr, cols, c * kChunk, tid, v);
#pragma unroll
            for (int i = 0; i < E; ++i) v[i] = exp2_full((v[i] - m) * kLog2e) * r;
            store_span<IO, VPL, THREADS, VEC>(yr, cols, c * kChunk, tid, v);
        }
    }
}

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

// Single-pass shapes (waves per row, vectors per lane), smallest first.
struct RegShape {
    int wpr, vpl;
};
constexpr RegShape kRegShapes[] = {{1, 1}, {1, 2}, {1, 4}, {1, 8},
                                   {2, 8}, {4, 8}, {8, 8}, {16, 8}};
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
    const void* fn = vec ? reinterpret_cast<const void*>(&softmax_reg_kernel<IO, WPR, VPL, true>)
                         : reinterpret_cast<const void*>(&softmax_reg_kernel<IO, WPR, VPL, false>);
    return launch_kernel(fn, grid, kThreads, s, x, y, rows, cols, ldx, ldy);
}

template <class IO>
hipError_t dispatch_reg(int shape, const void* x, void* y, int64_t rows, int64_t cols,
                        int64_t ldx, int64_t ldy, bool vec, hipStream_t s) {
    switch (shape) {
        case 0: return launch_reg<IO, 1, 1>(x, y, rows, cols, ldx, ldy, vec, s);
        case 1: return launch_reg<IO, 1, 2>(x, y, rows, cols, ldx, ldy, vec, s);
        case 2: return launch_reg<IO, 1, 4>(x, y, rows, cols, ldx, ldy, vec, s);
        case 3: return launch_reg<IO, 1, 8>(x, y, rows, cols, ldx, ldy, vec, s);
        case 4: return launch_reg<IO, 2, 8>(x, y, rows, cols, ldx, ldy, vec, s);
        case 5: return launch_reg<IO, 4, 8>(x, y, rows, cols, ldx, ldy, vec, s);
        case 6: return launch_reg<IO, 8, 8>(x, y, rows, cols, ldx, ldy, vec, s);
        default: return launch_reg<IO, 16, 8>(x, y, rows, cols, ldx, ldy, vec, s);
    }
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

template <class IO>
hipError_t launch_softmax_t(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t ldy, bool online, hipStream_t s) {
    const bool vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0 &&
                     (ldx * IO::kBytes) % 16 == 0 && (ldy * IO::kBytes) % 16 == 0;
    if (!online) {
        for (int i = 0; i < kNumRegShapes; ++i)
            if (cols <= reg_capacity<IO>(kRegShapes[i]))
                return dispatch_reg<IO>(i, x, y, rows, cols, ldx, ldy, vec, s);
    }
    return launch_online<IO>(x, y, rows, cols, ldx, ldy, vec, s);
}

}  // namespace

int64_t softmax_onchip_max_cols(Dtype dt) {
    return dt == kF32 ? reg_capacity<IoF32>(kRegShapes[kNumRegShapes - 1])
                      : reg_capacity<IoBF16>(kRegShapes[kNumRegShapes - 1]);
}

hipError_t launch_softmax(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                          int64_t ldy, Dtype dt, bool online, hipStream_t s) {
    return dt == kF32 ? launch_softmax_t<IoF32>(x, y, rows, cols, ldx, ldy, online, s)
                      : launch_softmax_t<IoBF16>(x, y, rows, cols, ldx, ldy, online, s);
}

}  // namespace fk
