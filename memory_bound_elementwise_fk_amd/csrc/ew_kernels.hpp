// ew_kernels.hpp -- streaming kernels that read every element once and
// write it once: tanh-GELU, the fused op chain and a plain byte copy (the
// bandwidth ceiling). gfx950, wave64.
//
// Tiling follows the masked-block scheme of the Triton tutorial page
// (accesspath.com, "Triton in practice"): ceil(n / TILE) tiles, each lane
// owning fixed offsets, and lanes past n neither loading nor storing. On
// MI355X each lane moves 16 bytes per load (global_load_dwordx4), so one
// wave instruction covers 1 KiB of consecutive HBM (eight 128-byte lines):
// the coalesced pattern of "Lecture 6: GPU Kernels and Triton", section 4.
// Full tiles run without masks; only the last tile masks vectors and
// finishes the < 16-byte scalar tail.
//
// Launch shape: one small tile per workgroup, dispatched in order, so the
// addresses in flight at any moment form one compact window of HBM; this
// measured faster on MI355X than persistent grid-stride loops over the same
// data (which spread the window) or larger per-lane batches.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace fk {

struct GeluOp {
    template <int N>
    __device__ inline void operator()(float (&v)[N]) const {
        gelu_tanh_n(v);
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
            } else if (k == kOpRelu) {
#pragma unroll
                for (int j = 0; j < N; ++j) v[j] = relu1(v[j]);
            } else {
                gelu_tanh_n(v);
            }
        }
    }
};

// The three-op chains "scalar op, activation, scalar op" (K0 and K2 each
// kOpAdd or kOpMul, K1 kOpGelu or kOpRelu; C3's 0.5 * GELU(x + 1) is one)
// with the op kinds fixed at compile time: straight-line code, which the
// compiler schedules across the three ops, instead of ChainOp's branch per op
// (measured 2-3 % faster on a 32 MiB chain, where each wave's arithmetic
// after its load returns adds to the kernel's latency). Same rounding as
// ChainOp: each op rounds to fp32.
template <int K0, int K1, int K2>
struct AffActAffOp {
    float s0, s2;
    template <int N>
    __device__ inline void operator()(float (&v)[N]) const {
#pragma unroll
        for (int j = 0; j < N; ++j) v[j] = K0 == kOpAdd ? v[j] + s0 : v[j] * s0;
        if constexpr (K1 == kOpGelu) {
            gelu_tanh_n(v);
        } else {
#pragma unroll
            for (int j = 0; j < N; ++j) v[j] = relu1(v[j]);
        }
#pragma unroll
        for (int j = 0; j < N; ++j) v[j] = K2 == kOpAdd ? v[j] + s2 : v[j] * s2;
    }
};

// Unpack U 16-byte words, apply the op to all their values at once, repack.
template <class IO, int U, class Op>
__device__ inline void ew_apply(u32x4 (&w)[U], const Op& op) {
    constexpr int V = IO::kVec;
    float v[U * V];
#pragma unroll
    for (int u = 0; u < U; ++u) IO::unpack(w[u], &v[u * V]);
    op(v);
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = IO::pack(&v[u * V]);
}

// The one ragged tile: whole vectors below nvec, then the scalar tail (the
// last n % V elements, fewer than V <= 8 < T).
template <class IO, int T, int U, bool NT, class Op>
__device__ inline void ew_ragged_tile(const u32x4* x, u32x4* y, int64_t n, int64_t nvec,
                                      int64_t v0, const Op& op) {
    constexpr int V = IO::kVec;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t vi = v0 + int64_t(u) * T;
        if (vi < nvec) {
            u32x4 w[1] = {ld16<NT>(x + vi)};
            ew_apply<IO, 1>(w, op);
            st16<NT>(y + vi, w[0]);
        }
    }
    const int64_t i = nvec * V + threadIdx.x;
    if (i < n) {
        float v[1] = {IO::load1(x, i)};
        op(v);
        IO::store1(y, i, v[0]);
    }
}

// x, y 16-byte aligned. Tile t covers vectors [t*T*U, (t+1)*T*U); lane l of
// the workgroup owns vectors t*T*U + u*T + l, u < U. The host passes nfull,
// the number of tiles without a ragged end (one tile more holds the ragged
// end when n is not a multiple of the tile). With STRIDED false there is
// exactly one workgroup per tile and no loop: with one 16-byte vector per
// lane a workgroup lives for a single load and store, so per-workgroup
// setup matters. STRIDED true loops over tiles (only for sizes past 2^31
// work-items). x == y (in place) is safe despite __restrict__: every
// address is loaded and stored by the same lane, and the store depends on
// the loaded value.
template <class IO, int T, int U, bool NT, bool STRIDED, class Op>
__global__ __launch_bounds__(T) void ew_vec_kernel(const u32x4* __restrict__ x,
                                                   u32x4* __restrict__ y, int64_t n,
                                                   int64_t nfull, Op op) {
    constexpr int64_t kTileVec = int64_t(T) * U;
    const int64_t ntiles = STRIDED ? (n + kTileVec * IO::kVec - 1) / (kTileVec * IO::kVec) : 0;
    for (int64_t tile = blockIdx.x;; tile += gridDim.x) {
        if constexpr (STRIDED) {
            if (tile >= ntiles) break;
        }
        const int64_t v0 = tile * kTileVec + threadIdx.x;
        if (tile < nfull) {
            u32x4 w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = ld16<NT>(x + v0 + u * T);
            ew_apply<IO, U>(w, op);
#pragma unroll
            for (int u = 0; u < U; ++u) st16<NT>(y + v0 + u * T, w[u]);
        } else {
            ew_ragged_tile<IO, T, U, NT>(x, y, n, n / IO::kVec, v0, op);
        }
        if constexpr (!STRIDED) break;
    }
}

// Any element-aligned x, y: one element per lane per step, still coalesced.
template <class IO, int T, int PER, class Op>
__global__ __launch_bounds__(T) void ew_scalar_kernel(const void* x, void* y, int64_t n, Op op) {
    constexpr int64_t kTile = int64_t(T) * PER;
    const int64_t ntiles = (n + kTile - 1) / kTile;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t base = tile * kTile + threadIdx.x;
        float v[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int64_t i = base + int64_t(u) * T;
            v[u] = i < n ? IO::load1(x, i) : 0.0f;
        }
        op(v);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int64_t i = base + int64_t(u) * T;
            if (i < n) IO::store1(y, i, v[u]);
        }
    }
}

// Byte copy: 16-byte body, then the < 16-byte tail one byte per lane.
template <int T, int U, bool NT>
__global__ __launch_bounds__(T) void copy_vec_kernel(const u32x4* __restrict__ x,
                                                     u32x4* __restrict__ y, int64_t nbytes) {
    constexpr int64_t kTileVec = int64_t(T) * U;
    const int64_t nvec = nbytes / 16;
    const int64_t nfull = nvec / kTileVec;
    const int64_t ntiles = (nbytes + kTileVec * 16 - 1) / (kTileVec * 16);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t v0 = tile * kTileVec + threadIdx.x;
        if (tile < nfull) {
            u32x4 w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = ld16<NT>(x + v0 + u * T);
#pragma unroll
            for (int u = 0; u < U; ++u) st16<NT>(y + v0 + u * T, w[u]);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t vi = v0 + int64_t(u) * T;
                if (vi < nvec) st16<NT>(y + vi, ld16<NT>(x + vi));
            }
            const int64_t b = nvec * 16 + threadIdx.x;
            if (b < nbytes)
                reinterpret_cast<uint8_t*>(y)[b] = reinterpret_cast<const uint8_t*>(x)[b];
        }
    }
}

template <int T>
__global__ __launch_bounds__(T) void copy_byte_kernel(const uint8_t* x, uint8_t* y,
                                                      int64_t nbytes) {
    const int64_t stride = int64_t(gridDim.x) * T;
    for (int64_t i = int64_t(blockIdx.x) * T + threadIdx.x; i < nbytes; i += stride) y[i] = x[i];
}

}  // namespace fk
