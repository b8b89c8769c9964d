// elementwise.hip -- streaming kernels that read every element once and
// write it once: tanh-GELU, the fused op chain, and a plain byte copy (the
// bandwidth ceiling). gfx950, wave64.
//
// Tiling follows the masked-block scheme of the Triton tutorial page
// (accesspath.com, "Triton in practice"): a grid of ceil(n / TILE) tiles,
// each lane owning fixed offsets, and lanes past n neither loading nor
// storing. On MI355X each lane moves 16 bytes per load (global_load_dwordx4),
// so one wave instruction covers 1 KiB of consecutive HBM (eight 128-byte
// lines): the coalesced pattern of "Lecture 6: GPU Kernels and Triton",
// section 4. A lane issues UNROLL such loads before it computes, which keeps
// enough bytes in flight to cover HBM latency. Full tiles run without masks;
// only the last tile masks vectors and finishes the < 16-byte scalar tail.
#include "device_common.hpp"
#include "launch.hpp"

namespace fk {
namespace {

constexpr int kEwThreads = 256;
constexpr int64_t kMaxGrid = int64_t(1) << 22;  // grid-stride beyond this

struct GeluOp {
    template <int N>
    __device__ inline void operator()(float (&v)[N]) const {
#pragma unroll
        for (int j = 0; j < N; ++j) v[j] = gelu_tanh(v[j]);
    }
};

// The ops run in list order on the lane's registers; the op kind is uniform
// across the launch, so the branches are scalar. Every op rounds to fp32
// (the library is built with FMA contraction off), which reproduces running
// each op as its own kernel.
struct ChainOp {
    OpList ops;
    template <int N>
    __device__ inline void operator()(float (&v)[N]) const {
        for (int i = 0; i < ops.n; ++i) {
            const int32_t k = ops.kind[i];
            const float s = ops.scalar[i];
            if (k == kOpAdd) {
#pragma unroll
                for (int j = 0; j < N; ++j) v[j] = v[j] + s;
            } else if (k == kOpMul) {
#pragma unroll
                for (int j = 0; j < N; ++j) v[j] = v[j] * s;
            } else {
#pragma unroll
                for (int j = 0; j < N; ++j) v[j] = gelu_tanh(v[j]);
            }
        }
    }
};

template <class IO, int UNROLL, bool NT, class Op>
__device__ inline void ew_ragged_tile(const u32x4* x, u32x4* y, int64_t n, int64_t nvec,
                                      int64_t v0, const Op& op) {
    constexpr int V = IO::kVec;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t vi = v0 + int64_t(u) * kEwThreads;
        if (vi < nvec) {
            float v[V];
            IO::unpack(ld16<NT>(x + vi), v);
            op(v);
            st16<NT>(y + vi, IO::pack(v));
        }
    }
    // scalar tail: the last n % V elements (fewer than V <= 8 < kEwThreads)
    const int64_t i = nvec * V + threadIdx.x;
    if (i < n) {
        float v[1] = {IO::load1(x, i)};
        op(v);
        IO::store1(y, i, v[0]);
    }
}

// x, y 16-byte aligned. Tile t covers vectors [t*T, (t+1)*T), T = 256*UNROLL;
// lane l of the WG owns vectors t*T + u*256 + l, u < UNROLL.
template <class IO, int UNROLL, bool NT, class Op>
__global__ __launch_bounds__(kEwThreads) void ew_vec_kernel(const u32x4* x, u32x4* y, int64_t n,
                                                            Op op) {
    constexpr int V = IO::kVec;
    constexpr int64_t kTileVec = int64_t(kEwThreads) * UNROLL;
    const int64_t nvec = n / V;
    const int64_t nfull = nvec / kTileVec;
    const int64_t ntiles = (n + kTileVec * V - 1) / (kTileVec * V);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t v0 = tile * kTileVec + threadIdx.x;
        if (tile < nfull) {
            u32x4 w[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) w[u] = ld16<NT>(x + v0 + u * kEwThreads);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                float v[V];
                IO::unpack(w[u], v);
                op(v);
                w[u] = IO::pack(v);
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) st16<NT>(y + v0 + u * kEwThreads, w[u]);
        } else {
            ew_ragged_tile<IO, UNROLL, NT>(x, y, n, nvec, v0, op);
        }
    }
}

// Any element-aligned x, y: one element per lane per step, still coalesced.
template <class IO, int PER, class Op>
__global__ __launch_bounds__(kEwThreads) void ew_scalar_kernel(const void* x, void* y, int64_t n,
                                                               Op op) {
    constexpr int64_t kTile = int64_t(kEwThreads) * PER;
    const int64_t ntiles = (n + kTile - 1) / kTile;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t base = tile * kTile + threadIdx.x;
        float v[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int64_t i = base + int64_t(u) * kEwThreads;
            v[u] = i < n ? IO::load1(x, i) : 0.0f;
        }
        op(v);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int64_t i = base + int64_t(u) * kEwThreads;
            if (i < n) IO::store1(y, i, v[u]);
        }
    }
}

// Byte copy: 16-byte body, then the < 16-byte tail one byte per lane.
template <int UNROLL, bool NT>
__global__ __launch_bounds__(kEwThreads) void copy_vec_kernel(const u32x4* x, u32x4* y,
                                                              int64_t nbytes) {
    constexpr int64_t kTileVec = int64_t(kEwThreads) * UNROLL;
    const int64_t nvec = nbytes / 16;
    const int64_t nfull = nvec / kTileVec;
    const int64_t ntiles = (nbytes + kTileVec * 16 - 1) / (kTileVec * 16);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t v0 = tile * kTileVec + threadIdx.x;
        if (tile < nfull) {
            u32x4 w[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) w[u] = ld16<NT>(x + v0 + u * kEwThreads);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) st16<NT>(y + v0 + u * kEwThreads, w[u]);
        } else {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int64_t vi = v0 + int64_t(u) * kEwThreads;
                if (vi < nvec) st16<NT>(y + vi, ld16<NT>(x + vi));
            }
            const int64_t b = nvec * 16 + threadIdx.x;
            if (b < nbytes)
                reinterpret_cast<uint8_t*>(y)[b] = reinterpret_cast<const uint8_t*>(x)[b];
        }
    }
}

__global__ __launch_bounds__(kEwThreads) void copy_byte_kernel(const uint8_t* x, uint8_t* y,
                                                               int64_t nbytes) {
    const int64_t stride = int64_t(gridDim.x) * kEwThreads;
    for (int64_t i = int64_t(blockIdx.x) * kEwThreads + threadIdx.x; i < nbytes; i += stride)
        y[i] = x[i];
}

// ----------------------------------------------------------------- launch -
template <class... Args>
hipError_t launch_kernel(const void* fn, int64_t grid, int block, hipStream_t s, Args... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(block), argv, 0, s);
}

int64_t grid_for(int64_t work_units) {
    return work_units < kMaxGrid ? (work_units > 0 ? work_units : 1) : kMaxGrid;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Lanes keep 64 bytes of fp32 or 32 bytes of bf16 loads in flight per tile.
template <class IO>
constexpr int kUnroll = IO::kBytes == 4 ? 4 : 2;
constexpr bool kNonTemporal = false;
constexpr int kScalarPer = 8;

template <class IO, class Op>
hipError_t launch_ew(const void* x, void* y, int64_t n, const Op& op, hipStream_t s) {
    if (aligned16(x) && aligned16(y)) {
        constexpr int U = kUnroll<IO>;
        const int64_t tile = int64_t(kEwThreads) * U * IO::kVec;
        return launch_kernel(reinterpret_cast<const void*>(&ew_vec_kernel<IO, U, kNonTemporal, Op>),
                             grid_for((n + tile - 1) / tile), kEwThreads, s,
                             static_cast<const u32x4*>(x), static_cast<u32x4*>(y), n, op);
    }
    const int64_t tile = int64_t(kEwThreads) * kScalarPer;
    return launch_kernel(reinterpret_cast<const void*>(&ew_scalar_kernel<IO, kScalarPer, Op>),
                         grid_for((n + tile - 1) / tile), kEwThreads, s, x, y, n, op);
}

}  // namespace

hipError_t launch_gelu(const void* x, void* y, int64_t n, Dtype dt, hipStream_t s) {
    return dt == kF32 ? launch_ew<IoF32>(x, y, n, GeluOp{}, s)
                      : launch_ew<IoBF16>(x, y, n, GeluOp{}, s);
}

hipError_t launch_chain(const void* x, void* y, int64_t n, Dtype dt, const OpList& ops,
                        hipStream_t s) {
    const ChainOp op{ops};
    return dt == kF32 ? launch_ew<IoF32>(x, y, n, op, s) : launch_ew<IoBF16>(x, y, n, op, s);
}

hipError_t launch_copy(const void* x, void* y, int64_t nbytes, hipStream_t s) {
    if (aligned16(x) && aligned16(y)) {
        constexpr int U = 4;
        const int64_t tile = int64_t(kEwThreads) * U * 16;
        return launch_kernel(reinterpret_cast<const void*>(&copy_vec_kernel<U, kNonTemporal>),
                             grid_for((nbytes + tile - 1) / tile), kEwThreads, s,
                             static_cast<const u32x4*>(x), static_cast<u32x4*>(y), nbytes);
    }
    return launch_kernel(reinterpret_cast<const void*>(&copy_byte_kernel),
                         grid_for((nbytes + kEwThreads * 16 - 1) / (kEwThreads * 16)), kEwThreads,
                         s, static_cast<const uint8_t*>(x), static_cast<uint8_t*>(y), nbytes);
}

}  // namespace fk
