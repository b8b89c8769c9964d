// layernorm_kernels.hpp -- fused LayerNorm row kernel for gfx950, with an
// optional tanh-GELU epilogue.
//
// LayerNorm is the first kernel of the LayerNorm -> Linear -> GELU example
// of "Lecture 6: GPU Kernels and Triton", section 6.1, whose point is that
// the fused version reads x once and writes the result once, keeping the
// intermediates in registers. Per row (standard definition; the page gives
// no formula): mu = mean(x), var = mean((x - mu)^2) (biased),
// y = (x - mu) / sqrt(var + eps) * gamma + beta, then y = GELU(y) if asked.
//
// The row is held in the VGPRs of its lanes (same shapes as the single-pass
// softmax), so HBM is read once and written once. Statistics use the
// corrected two-pass scheme over registers: mu = sum(x) / n, then
// d = x - mu, a = sum(d), q = sum(d^2), c = a / n, var = q / n - c^2 and the
// output uses (d - c); the correction c removes the rounding of mu, so the
// error does not grow with |mu| (rows shifted far from 0). Reductions are
// lane-local, DPP across the wave, LDS across the row's waves, in a fixed
// order (bitwise reproducible).
#pragma once

#include "softmax_kernels.hpp"

namespace fk {

// Multiply by gamma and add beta, column by column, in load_span's layout.
// gamma / beta are per-column arrays of the row dtype, or null (1 / 0).
template <class IO, int VPL, int LANES, bool VEC>
__device__ inline void affine_span(const char* gp, const char* bp, int64_t cols, int lane,
                                   float (&v)[VPL * IO::kVec]) {
    constexpr int V = IO::kVec;
    if constexpr (VEC) {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int64_t c = (int64_t(k) * LANES + lane) * V;
            float g[V] = {}, b[V] = {};
            if (c + V <= cols) {
                if (gp) IO::unpack(ld16<false>(reinterpret_cast<const u32x4*>(gp + c * IO::kBytes)), g);
                if (bp) IO::unpack(ld16<false>(reinterpret_cast<const u32x4*>(bp + c * IO::kBytes)), b);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    g[e] = (gp && c + e < cols) ? IO::load1(gp, c + e) : 1.0f;
                    b[e] = (bp && c + e < cols) ? IO::load1(bp, c + e) : 0.0f;
                }
            }
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if (gp) v[k * V + e] *= g[e];
                if (bp) v[k * V + e] += b[e];
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < VPL * V; ++k) {
            const int64_t c = int64_t(k) * LANES + lane;
            if (c < cols) {
                if (gp) v[k] *= IO::load1(gp, c);
                if (bp) v[k] += IO::load1(bp, c);
            }
        }
    }
}

template <class IO, int WPR, int VPL, bool VEC, bool NT = false>
__global__ __launch_bounds__(reg_threads<WPR>()) void layernorm_reg_kernel(
    const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy,
    const void* gamma, const void* beta, float eps, int gelu) {
    constexpr int V = IO::kVec;
    constexpr int E = VPL * V;
    constexpr int kRowLanes = WPR * kWave;
    constexpr int kRowsPerWg = reg_threads<WPR>() / kRowLanes;
    __shared__ float red[2][kRowsPerWg * WPR];

    const int sub = threadIdx.x / kRowLanes;
    const int lr = threadIdx.x % kRowLanes;
    const int wave = lr / kWave;
    const int lane = threadIdx.x % kWave;
    const bool full = cols >= int64_t(kRowLanes) * E;  // every value of every lane is a column
    const float n = static_cast<float>(cols);
    const char* gp = static_cast<const char*>(gamma);
    const char* bp = static_cast<const char*>(beta);

    for (int64_t rb = int64_t(blockIdx.x) * kRowsPerWg; rb < rows;
         rb += int64_t(gridDim.x) * kRowsPerWg) {
        const int64_t row = rb + sub;
        const bool active = row < rows;
        float v[E];
        if (active) {
            load_span<IO, VPL, kRowLanes, VEC, NT>(row_ptr<IO>(x, row, ldx), cols, 0, lr, v, 0.0f);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i) v[i] = 0.0f;
        }

        // mean
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < E; ++i) s += v[i];
        s = wave_sum(s);
        if constexpr (WPR > 1) {
            if (lane == 0) red[0][sub * WPR + wave] = s;
            __syncthreads();
            s = red[0][sub * WPR];
#pragma unroll
            for (int w = 1; w < WPR; ++w) s += red[0][sub * WPR + w];
            __syncthreads();
        }
        const float mu = s / n;

        // deviations, their sum (the correction) and their squares
        float a = 0.0f, q = 0.0f;
#pragma unroll
        for (int i = 0; i < E; ++i) {
            float d = v[i] - mu;
            if (!full && span_col<IO, kRowLanes, VEC>(i, lr) >= cols) d = 0.0f;
            v[i] = d;
            a += d;
            q = fmaf(d, d, q);
        }
        a = wave_sum(a);
        q = wave_sum(q);
        if constexpr (WPR > 1) {
            if (lane == 0) {
                red[0][sub * WPR + wave] = a;
                red[1][sub * WPR + wave] = q;
            }
            __syncthreads();
            a = red[0][sub * WPR];
            q = red[1][sub * WPR];
#pragma unroll
            for (int w = 1; w < WPR; ++w) {
                a += red[0][sub * WPR + w];
                q += red[1][sub * WPR + w];
            }
            __syncthreads();
        }
        const float c = a / n;
        const float var = fmaxf(q / n - c * c, 0.0f);
        const float rstd = 1.0f / sqrtf(var + eps);

        // normalise, affine, optional GELU, write back
#pragma unroll
        for (int i = 0; i < E; ++i) v[i] = (v[i] - c) * rstd;
        if (gp || bp) affine_span<IO, VPL, kRowLanes, VEC>(gp, bp, cols, lr, v);
        if (gelu) gelu_tanh_n(v);
        if (active)
            store_span<IO, VPL, kRowLanes, VEC, NT>(row_ptr<IO>(y, row, ldy), cols, 0, lr, v);
    }
}

}  // namespace fk
