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
// output is (d - c) rstd, formed as fma(d, rstd, -c rstd); the correction c
// removes the rounding of mu, so the error does not grow with |mu| (rows
// shifted far from 0). The divisions by n are products with 1/n (rounded
// once per launch; exact for powers of two) and rstd is the hardware
// reciprocal square root (v_rsq_f32, about 1 ulp): the IEEE divisions and
// square root took ~90 of the ~380 VALU instructions a lane issues per
// 4096-column bf16 row with GELU (16 values per lane). Reductions
// are lane-local, DPP across the wave, LDS across the row's waves, in a
// fixed order (bitwise reproducible). gamma and beta are loaded before the
// row's statistics (not after them, where their latency would add to every
// row's) and applied with one more fma.
#pragma once

#include "softmax_kernels.hpp"

namespace fk {

// gamma and beta of value chunk k of a lane (values k*V .. k*V+V-1 in
// load_span's layout; 1 and 0 where absent or past the row end).
template <class IO, int LANES, bool VEC>
__device__ inline void affine_chunk(const char* gp, const char* bp, int64_t cols, int lane, int k,
                                    float (&g)[IO::kVec], float (&b)[IO::kVec]) {
    constexpr int V = IO::kVec;
    if constexpr (VEC) {
        const int64_t c0 = (int64_t(k) * LANES + lane) * V;
        if (c0 + V <= cols) {
            if (gp) IO::unpack(ld16<false>(reinterpret_cast<const u32x4*>(gp + c0 * IO::kBytes)), g);
            else
#pragma unroll
                for (int e = 0; e < V; ++e) g[e] = 1.0f;
            if (bp) IO::unpack(ld16<false>(reinterpret_cast<const u32x4*>(bp + c0 * IO::kBytes)), b);
            else
#pragma unroll
                for (int e = 0; e < V; ++e) b[e] = 0.0f;
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const int64_t col = span_col<IO, LANES, VEC>(k * V + e, lane);
        g[e] = (gp && col < cols) ? IO::load1(gp, col) : 1.0f;
        b[e] = (bp && col < cols) ? IO::load1(bp, col) : 0.0f;
    }
}

// gamma and beta are held in registers (loaded once per workgroup, before
// the first row, so their latency overlaps the row loads) up to this many
// vectors per lane; wider shapes load them vector by vector in the
// epilogue, which keeps the register count of the widest rows bounded.
constexpr int kLnHoldAffineVpl = 2;

// Waves per SIMD the registers are budgeted for: two workgroups per CU where
// a workgroup of more than 8 waves would otherwise run alone (12 waves leave
// each SIMD 3), provided that costs at most 80 VGPRs (6 waves), gamma and
// beta are held (VPL <= 2) and the row is full (the masks of other widths
// would spill: measured 1.4-2x slower); 1 (no constraint) otherwise.
template <int WPR, int VPL, int FIT>
constexpr int ln_min_waves() {
    constexpr int per_simd = (reg_threads<WPR>() / kWave + 3) / 4;
    return (FIT == kFitFull && VPL <= kLnHoldAffineVpl && per_simd > 2 && 2 * per_simd <= 6)
               ? 2 * per_simd
               : 1;
}

// FIT (kFitAny, kFitVec, kFitFull) is what the launcher guarantees about the
// width: kFitFull (cols == WPR * 64 * VPL * V on the vector layout) compiles
// no masks; kFitVec (cols a multiple of V on the vector layout) masks whole
// vectors with tests that do not depend on the row; kFitAny masks values.
template <class IO, int WPR, int VPL, bool VEC, bool GELU, bool NT = false, int FIT = kFitAny>
__global__ __launch_bounds__(reg_threads<WPR>())
__attribute__((amdgpu_waves_per_eu(ln_min_waves<WPR, VPL, FIT>()))) void layernorm_reg_kernel(
    const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy,
    const void* gamma, const void* beta, float eps) {
    constexpr int V = IO::kVec;
    constexpr int E = VPL * V;
    constexpr int kRowLanes = WPR * kWave;
    constexpr int kRowsPerWg = reg_threads<WPR>() / kRowLanes;
    constexpr bool kHold = VPL <= kLnHoldAffineVpl;
    // partial sums of the row's waves: [parity][sum x, sum d, sum d^2][row, wave].
    // Consecutive rows of a workgroup use alternate halves, so each
    // reduction needs one barrier: a half is rewritten two rows later, after
    // every wave has passed the barriers of the row in between.
    __shared__ float red[2][3][kRowsPerWg * WPR];

    const int sub = threadIdx.x / kRowLanes;
    const int lr = threadIdx.x % kRowLanes;
    const int wave = lr / kWave;
    const int lane = threadIdx.x % kWave;
    const int slot = sub * WPR;
    static_assert(FIT == kFitAny || VEC, "fitted rows are a vector-layout case");
    constexpr bool kFull = FIT == kFitFull;
    constexpr bool kVfit = FIT == kFitVec;
    // the column count as the masked helpers see it: a compile-time constant
    // for full rows, so their masked paths fold away
    const int64_t span_cols = kFull ? int64_t(kRowLanes) * E : cols;
    const bool full = span_cols >= int64_t(kRowLanes) * E;  // every value of every lane is a column
    // kFitVec: which of this lane's vectors are columns (the same for every row)
    bool in_row[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) in_row[k] = (int64_t(k) * kRowLanes + lr) * V < cols;
    const float inv_n = 1.0f / static_cast<float>(cols);
    const char* gp = static_cast<const char*>(gamma);
    const char* bp = static_cast<const char*>(beta);

    // this lane's gamma and beta (1 and 0 where absent; columns past the row
    // end are computed but never stored, so their values do not matter)
    float g[kHold ? E : 1], b[kHold ? E : 1];
    if constexpr (kHold) {
        if constexpr (kVfit) {
            if (gp) load_span_vfit<IO, VPL, kRowLanes>(gp, cols, lr, g, 1.0f);
            if (bp) load_span_vfit<IO, VPL, kRowLanes>(bp, cols, lr, b, 0.0f);
            if (!gp) {
#pragma unroll
                for (int i = 0; i < E; ++i) g[i] = 1.0f;
            }
            if (!bp) {
#pragma unroll
                for (int i = 0; i < E; ++i) b[i] = 0.0f;
            }
        } else if (gp && bp) {
            load_span2<IO, VPL, kRowLanes, VEC>(gp, bp, span_cols, 0, lr, g, b, 0.0f);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i) {
                g[i] = 1.0f;
                b[i] = 0.0f;
            }
            if (gp) load_span<IO, VPL, kRowLanes, VEC>(gp, span_cols, 0, lr, g, 1.0f);
            if (bp) load_span<IO, VPL, kRowLanes, VEC>(bp, span_cols, 0, lr, b, 0.0f);
        }
    }

    int par = 0;
    for (int64_t rb = int64_t(blockIdx.x) * kRowsPerWg; rb < rows;
         rb += int64_t(gridDim.x) * kRowsPerWg, par ^= 1) {
        const int64_t row = rb + sub;
        // one row per workgroup: rb < rows is the loop condition
        const bool active = kRowsPerWg == 1 || row < rows;
        float v[E];
        if (active) {
            if constexpr (kVfit)
                load_span_vfit<IO, VPL, kRowLanes, NT>(row_ptr<IO>(x, row, ldx), cols, lr, v, 0.0f);
            else
                load_span<IO, VPL, kRowLanes, VEC, NT>(row_ptr<IO>(x, row, ldx), span_cols, 0, lr,
                                                      v, 0.0f);
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
            if (lane == 0) red[par][0][slot + wave] = s;
            __syncthreads();
            s = red[par][0][slot];
#pragma unroll
            for (int w = 1; w < WPR; ++w) s += red[par][0][slot + w];
        }
        const float mu = s * inv_n;

        // deviations, their sum (the correction) and their squares; columns
        // past the row end (only in a ragged row) contribute 0
        float a = 0.0f, q = 0.0f;
        if (kVfit) {
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const float d = in_row[i / V] ? v[i] - mu : 0.0f;
                v[i] = d;
                a += d;
                q = fmaf(d, d, q);
            }
        } else if (full) {
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const float d = v[i] - mu;
                v[i] = d;
                a += d;
                q = fmaf(d, d, q);
            }
        } else {
            // rows held on chip are at most 65536 columns: 32-bit columns
            const int ncols = static_cast<int>(cols);
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const int col = static_cast<int>(span_col<IO, kRowLanes, VEC>(i, lr));
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
                red[par][1][slot + wave] = a;
                red[par][2][slot + wave] = q;
            }
            __syncthreads();
            a = red[par][1][slot];
            q = red[par][2][slot];
#pragma unroll
            for (int w = 1; w < WPR; ++w) {
                a += red[par][1][slot + w];
                q += red[par][2][slot + w];
            }
        }
        const float c = a * inv_n;
        const float var = fmaxf(fmaf(-c, c, q * inv_n), 0.0f);
        const float rstd = __builtin_amdgcn_rsqf(var + eps);
        const float off = -c * rstd;  // (d - c) rstd = d rstd + off

        // normalise, gamma and beta (two fused multiply-adds), optional GELU,
        // one chunk of V values (a 16-byte vector on the vector layout) at a
        // time, in place; then the row is stored
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float gk[V], bk[V];
            if constexpr (kHold) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    gk[e] = g[k * V + e];
                    bk[e] = b[k * V + e];
                }
            } else {
                affine_chunk<IO, kRowLanes, VEC>(gp, bp, span_cols, lr, k, gk, bk);
            }
            float t[V];
#pragma unroll
            for (int e = 0; e < V; ++e) t[e] = fmaf(fmaf(v[k * V + e], rstd, off), gk[e], bk[e]);
            if constexpr (GELU) gelu_tanh_n(t);
#pragma unroll
            for (int e = 0; e < V; ++e) v[k * V + e] = t[e];
        }
        if (active) {
            if constexpr (kVfit)
                store_span_vfit<IO, VPL, kRowLanes, NT>(row_ptr<IO>(y, row, ldy), cols, lr, v);
            else
                store_span<IO, VPL, kRowLanes, VEC, NT>(row_ptr<IO>(y, row, ldy), span_cols, 0, lr,
                                                       v);
        }
    }
}

}  // namespace fk
