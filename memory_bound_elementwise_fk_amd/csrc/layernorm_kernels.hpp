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

template <class IO, int WPR, int VPL, bool VEC, bool GELU, bool NT = false>
__global__ __launch_bounds__(reg_threads<WPR>()) void layernorm_reg_kernel(
    const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy,
    const void* gamma, const void* beta, float eps) {
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

        // deviations, their sum (the correction) and their squares; columns
        // past the row end (only in a ragged row) contribute 0
        float a = 0.0f, q = 0.0f;
        if (full) {
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const float d = v[i] - mu;
                v[i] = d;
                a += d;
                q = fmaf(d, d, q);
            }
        } else {
            const int ncols = static_cast<int>(cols);
#pragma unroll
            for (int i = 0; i < E; ++i) {
                // column of value i: vector layout (i / V * lanes + lane) * V + i % V,
                // scalar layout i * lanes + lane
                const int col = VEC ? ((i / V) * kRowLanes + lr) * V + i % V : i * kRowLanes + lr;
                const float d = col < ncols ? v[i] - mu : 0.0f;
                v[i] = d;
                a += d;
                q = fmaf(d, d, q);
            }
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

        // normalise, gamma and beta, optional GELU, write back -- one
        // 16-byte vector (or, on the scalar layout, eight values) at a time,
        // which keeps the epilogue's temporaries to one vector of registers
        char* yr = row_ptr<IO>(y, row, ldy);
        constexpr int kChunk = VEC ? V : (E < 8 ? E : 8);  // divides E (E = VPL * V)
        static_assert(E % kChunk == 0, "chunks cover the lane's values");
        // columns of value e of chunk k: c0 + e (vector layout: one 16-byte
        // vector) or c0 + e * kRowLanes (scalar layout); rows held on chip
        // are at most 65536 columns, so 32-bit column indices suffice
        constexpr int kStep = VEC ? 1 : kRowLanes;
        const int ncols = static_cast<int>(cols);
#pragma unroll
        for (int k = 0; k < E / kChunk; ++k) {
            const int c0 = VEC ? (k * kRowLanes + lr) * V : k * kChunk * kRowLanes + lr;
            float t[kChunk], gv[kChunk], bv[kChunk];
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                t[e] = (v[k * kChunk + e] - c) * rstd;
                gv[e] = 1.0f;
                bv[e] = 0.0f;
            }
            const bool whole = VEC && c0 + kChunk <= ncols;  // an unmasked 16-byte vector
            if (whole) {
                if (gp) IO::unpack(ld16<false>(reinterpret_cast<const u32x4*>(gp + int64_t(c0) * IO::kBytes)), gv);
                if (bp) IO::unpack(ld16<false>(reinterpret_cast<const u32x4*>(bp + int64_t(c0) * IO::kBytes)), bv);
            } else {
#pragma unroll
                for (int e = 0; e < kChunk; ++e) {
                    const int col = c0 + e * kStep;
                    if (gp && col < ncols) gv[e] = IO::load1(gp, col);
                    if (bp && col < ncols) bv[e] = IO::load1(bp, col);
                }
            }
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                if (gp) t[e] *= gv[e];
                if (bp) t[e] += bv[e];
            }
            if constexpr (GELU) gelu_tanh_n(t);
            if (!active) continue;
            if (whole) {
                st16<NT>(reinterpret_cast<u32x4*>(yr + int64_t(c0) * IO::kBytes), IO::pack(t));
            } else {
#pragma unroll
                for (int e = 0; e < kChunk; ++e) {
                    const int col = c0 + e * kStep;
                    if (col < ncols) IO::store1(yr, col, t[e]);
                }
            }
        }
    }
}

}  // namespace fk
