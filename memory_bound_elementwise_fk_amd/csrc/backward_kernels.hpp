// backward_kernels.hpp -- backward (gradient) kernels of the GELU and the row
// softmax, for gfx950. The pages print no backward formulas; both are the
// derivatives of the forward definitions (tanh-GELU of the "CS336 lecture 6"
// notes, section 4.2; row softmax of section 5.2):
//   GELU:    dx = dy * GELU'(x)                       (two reads, one write)
//   softmax: dx_j = y_j (dy_j - sum_k y_k dy_k)        (two reads, one write)
// Both are memory-bound like their forward kernels and use the same tiling:
// one 16-byte vector per lane per operand, and rows held in registers.
#pragma once

#include "ew_kernels.hpp"
#include "softmax_kernels.hpp"

namespace fk {

struct GeluBwdOp {
    template <int N>
    __device__ inline void operator()(const float (&x)[N], float (&g)[N]) const {
        gelu_tanh_grad_n(x, g);
    }
};

// out[i] = op(a[i], b[i]) with a, b, out 16-byte aligned; tiles of T vectors
// as in ew_vec_kernel (exactly one workgroup per tile unless STRIDED). out
// may be a or b exactly (every address is read and written by one lane).
template <class IO, int T, bool NT, bool STRIDED, class Op>
__global__ __launch_bounds__(T) void ew2_vec_kernel(const u32x4* __restrict__ a,
                                                    const u32x4* __restrict__ b,
                                                    u32x4* __restrict__ out, int64_t n,
                                                    int64_t nfull, Op op) {
    constexpr int V = IO::kVec;
    const int64_t ntiles = STRIDED ? (n + int64_t(T) * V - 1) / (int64_t(T) * V) : 0;
    for (int64_t tile = blockIdx.x;; tile += gridDim.x) {
        if constexpr (STRIDED) {
            if (tile >= ntiles) break;
        }
        const int64_t vi = tile * T + threadIdx.x;
        const int64_t nvec = n / V;
        if (tile < nfull || vi < nvec) {
            const u32x4 wa = ld16<NT>(a + vi);
            const u32x4 wb = ld16<NT>(b + vi);
            float va[V], vb[V];
            IO::unpack(wa, va);
            IO::unpack(wb, vb);
            op(va, vb);
            st16<NT>(out + vi, IO::pack(vb));
        }
        if (tile >= nfull) {  // the ragged tile: the last n % V elements
            const int64_t i = nvec * V + threadIdx.x;
            if (i < n) {
                float va[1] = {IO::load1(a, i)};
                float vb[1] = {IO::load1(b, i)};
                op(va, vb);
                IO::store1(out, i, vb[0]);
            }
        }
        if constexpr (!STRIDED) break;
    }
}

// Any element-aligned a, b, out: one element per lane per step.
template <class IO, int T, int PER, class Op>
__global__ __launch_bounds__(T) void ew2_scalar_kernel(const void* a, const void* b, void* out,
                                                       int64_t n, Op op) {
    constexpr int64_t kTile = int64_t(T) * PER;
    const int64_t ntiles = (n + kTile - 1) / kTile;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t base = tile * kTile + threadIdx.x;
        float va[PER], vb[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int64_t i = base + int64_t(u) * T;
            va[u] = i < n ? IO::load1(a, i) : 0.0f;
            vb[u] = i < n ? IO::load1(b, i) : 0.0f;
        }
        op(va, vb);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int64_t i = base + int64_t(u) * T;
            if (i < n) IO::store1(out, i, vb[u]);
        }
    }
}

// Softmax backward over rows held in registers (same shapes and reductions
// as softmax_reg_kernel): dot = sum y dy, dx = y (dy - dot). dx may be y or
// dy exactly (with the same stride): every value is in registers before the
// row is written.
// FIT: what the launcher guarantees about the width (kFitFull: no masking
// code; kFitVec: masks per vector; kFitAny: per value).
template <class IO, int WPR, int VPL, bool VEC, bool NT = false, int FIT = kFitAny>
__global__ __launch_bounds__(reg_threads<WPR>()) void softmax_bwd_reg_kernel(
    const void* y, const void* dy, void* dx, int64_t rows, int64_t cols, int64_t ldy,
    int64_t lddy, int64_t lddx) {
    constexpr int E = VPL * IO::kVec;
    constexpr int kRowLanes = WPR * kWave;
    constexpr int kRowsPerWg = reg_threads<WPR>() / kRowLanes;
    static_assert(FIT == kFitAny || VEC, "fitted rows are a vector-layout case");
    const int64_t span_cols = FIT == kFitFull ? int64_t(kRowLanes) * E : cols;
    // per-wave partial dot products, alternating halves row by row: one
    // barrier per row (a half is rewritten two rows later, after every wave
    // has passed the barrier of the row in between)
    __shared__ float red[2][kRowsPerWg * WPR];
    int par = 0;

    const int sub = threadIdx.x / kRowLanes;
    const int lr = threadIdx.x % kRowLanes;
    const int wave = lr / kWave;
    const int lane = threadIdx.x % kWave;

    for (int64_t rb = int64_t(blockIdx.x) * kRowsPerWg; rb < rows;
         rb += int64_t(gridDim.x) * kRowsPerWg, par ^= 1) {
        const int64_t row = rb + sub;
        const bool active = row < rows;
        float vy[E], vg[E];
        if (active) {
            if constexpr (FIT == kFitVec)
                load_span2_vfit<IO, VPL, kRowLanes, NT>(row_ptr<IO>(y, row, ldy),
                                                        row_ptr<IO>(dy, row, lddy), cols, lr, vy,
                                                        vg);
            else
                load_span2<IO, VPL, kRowLanes, VEC, NT>(row_ptr<IO>(y, row, ldy),
                                                        row_ptr<IO>(dy, row, lddy), span_cols, 0,
                                                        lr, vy, vg, 0.0f);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i) vy[i] = vg[i] = 0.0f;
        }
        float d = 0.0f;
#pragma unroll
        for (int i = 0; i < E; ++i) d = fmaf(vy[i], vg[i], d);
        d = wave_sum(d);
        if constexpr (WPR > 1) {
            if (lane == 0) red[par][sub * WPR + wave] = d;
            __syncthreads();
            d = red[par][sub * WPR];
#pragma unroll
            for (int w = 1; w < WPR; ++w) d += red[par][sub * WPR + w];
        }
#pragma unroll
        for (int i = 0; i < E; ++i) vg[i] = vy[i] * (vg[i] - d);
        if (active) {
            if constexpr (FIT == kFitVec)
                store_span_vfit<IO, VPL, kRowLanes, NT>(row_ptr<IO>(dx, row, lddx), cols, lr, vg);
            else
                store_span<IO, VPL, kRowLanes, VEC, NT>(row_ptr<IO>(dx, row, lddx), span_cols, 0,
                                                        lr, vg);
        }
    }
}

}  // namespace fk
