// softmax_kernels.hpp -- row softmax kernels for gfx950.
//
// The operation, per row: m = max_j x_j; s = sum_j exp(x_j - m);
// y_j = exp(x_j - m) / s ("CS336 lecture 6" notes, section 5.2: one block
// per row, load the row on chip, max, exponentials and sum, normalise,
// write back). Numerators are e'_j = 2^((x_j - m) log2e + 8) and the
// divisor is the sum of the same e'_j, so the factor 2^8 cancels exactly
// and the numerators stay normal down to 2^-134 (softmax_numerator). The
// max element gives exactly 2^8, so a one-column row is exactly 1 and a
// constant row of 2^k columns exactly 2^-k.
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
// e' / (l 2^8).
#pragma once

#include "device_common.hpp"

namespace fk {

constexpr float kNegInf = -__builtin_inff();

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
// layout: columns k*LANES + lane. Columns >= cols read as `fill` (-inf for
// the max/exp reductions, 0 for sums). A span that lies entirely inside the
// row (a uniform test) takes the unmasked path, whose loads are all issued
// before any of them is unpacked: left to itself the instruction scheduler
// interleaves the unpacking with the loads and waits for each load before
// issuing the next, which serialises their HBM latencies.
template <class IO, int VPL, int LANES, bool VEC, bool NT = false>
__device__ inline void load_span(const char* xr, int64_t cols, int64_t c0, int lane,
                                 float (&v)[VPL * IO::kVec], float fill = -__builtin_inff()) {
    constexpr int V = IO::kVec;
    constexpr int64_t kSpan = int64_t(VPL) * LANES * V;
    if constexpr (VEC) {
        if (cols - c0 >= kSpan) {
            u32x4 w[VPL];
#pragma unroll
            for (int k = 0; k < VPL; ++k)
                w[k] = ld16<NT>(reinterpret_cast<const u32x4*>(
                    xr + (c0 + (int64_t(k) * LANES + lane) * V) * IO::kBytes));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < VPL; ++k) IO::unpack(w[k], &v[k * V]);
            return;
        }
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int64_t c = c0 + (int64_t(k) * LANES + lane) * V;
            if (c + V <= cols) {
                IO::unpack(ld16<NT>(reinterpret_cast<const u32x4*>(xr + c * IO::kBytes)),
                           &v[k * V]);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    v[k * V + e] = (c + e < cols) ? IO::load1(xr, c + e) : fill;
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < VPL * V; ++k) {
            const int64_t c = c0 + int64_t(k) * LANES + lane;
            v[k] = c < cols ? IO::load1(xr, c) : fill;
        }
    }
}

// Two spans of the same columns from two rows (e.g. y and dy): on the
// unmasked path all loads of both are in flight before any is unpacked.
template <class IO, int VPL, int LANES, bool VEC, bool NT = false>
__device__ inline void load_span2(const char* ar, const char* br, int64_t cols, int64_t c0,
                                  int lane, float (&va)[VPL * IO::kVec],
                                  float (&vb)[VPL * IO::kVec], float fill) {
    constexpr int V = IO::kVec;
    constexpr int64_t kSpan = int64_t(VPL) * LANES * V;
    if constexpr (VEC) {
        if (cols - c0 >= kSpan) {
            u32x4 wa[VPL], wb[VPL];
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                const int64_t off = (c0 + (int64_t(k) * LANES + lane) * V) * IO::kBytes;
                wa[k] = ld16<NT>(reinterpret_cast<const u32x4*>(ar + off));
                wb[k] = ld16<NT>(reinterpret_cast<const u32x4*>(br + off));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                IO::unpack(wa[k], &va[k * V]);
                IO::unpack(wb[k], &vb[k * V]);
            }
            return;
        }
    }
    load_span<IO, VPL, LANES, VEC, NT>(ar, cols, c0, lane, va, fill);
    load_span<IO, VPL, LANES, VEC, NT>(br, cols, c0, lane, vb, fill);
}

// Column (relative to the span start) of value i of a lane in load_span's
// layout.
template <class IO, int LANES, bool VEC>
__device__ inline int64_t span_col(int i, int lane) {
    constexpr int V = IO::kVec;
    if constexpr (VEC) return (int64_t(i / V) * LANES + lane) * V + i % V;
    else return int64_t(i) * LANES + lane;
}

template <class IO, int VPL, int LANES, bool VEC, bool NT = false>
__device__ inline void store_span(char* yr, int64_t cols, int64_t c0, int lane,
                                  const float (&v)[VPL * IO::kVec]) {
    constexpr int V = IO::kVec;
    constexpr int64_t kSpan = int64_t(VPL) * LANES * V;
    if constexpr (VEC) {
        if (cols - c0 >= kSpan) {
#pragma unroll
            for (int k = 0; k < VPL; ++k)
                st16<NT>(reinterpret_cast<u32x4*>(
                             yr + (c0 + (int64_t(k) * LANES + lane) * V) * IO::kBytes),
                         IO::pack(&v[k * V]));
            return;
        }
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int64_t c = c0 + (int64_t(k) * LANES + lane) * V;
            if (c + V <= cols) {
                st16<NT>(reinterpret_cast<u32x4*>(yr + c * IO::kBytes), IO::pack(&v[k * V]));
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

// A row whose width is a multiple of V, on the vector layout: each of a
// lane's vectors lies wholly inside or wholly outside the row, so a mask is
// one test per vector, the same for every row. All loads of the span are
// issued before any is unpacked (as on the unmasked path); vectors past the
// row end read as `fill`.
template <class IO, int VPL, int LANES, bool NT = false>
__device__ inline void load_span_vfit(const char* xr, int64_t cols, int lane,
                                      float (&v)[VPL * IO::kVec], float fill) {
    constexpr int V = IO::kVec;
    u32x4 w[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int64_t c = (int64_t(k) * LANES + lane) * V;
        w[k] = c < cols ? ld16<NT>(reinterpret_cast<const u32x4*>(xr + c * IO::kBytes))
                        : u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        IO::unpack(w[k], &v[k * V]);
        if ((int64_t(k) * LANES + lane) * V >= cols) {
#pragma unroll
            for (int e = 0; e < V; ++e) v[k * V + e] = fill;
        }
    }
}

// Two rows' spans (e.g. y and dy) on the same columns, all loads of both in
// flight before any is unpacked; vectors past the row end read as 0.
template <class IO, int VPL, int LANES, bool NT = false>
__device__ inline void load_span2_vfit(const char* ar, const char* br, int64_t cols, int lane,
                                       float (&va)[VPL * IO::kVec], float (&vb)[VPL * IO::kVec]) {
    constexpr int V = IO::kVec;
    u32x4 wa[VPL], wb[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int64_t c = (int64_t(k) * LANES + lane) * V;
        const bool in = c < cols;
        wa[k] = in ? ld16<NT>(reinterpret_cast<const u32x4*>(ar + c * IO::kBytes))
                   : u32x4{0u, 0u, 0u, 0u};
        wb[k] = in ? ld16<NT>(reinterpret_cast<const u32x4*>(br + c * IO::kBytes))
                   : u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        IO::unpack(wa[k], &va[k * V]);
        IO::unpack(wb[k], &vb[k * V]);
    }
}

template <class IO, int VPL, int LANES, bool NT = false>
__device__ inline void store_span_vfit(char* yr, int64_t cols, int lane,
                                       const float (&v)[VPL * IO::kVec]) {
    constexpr int V = IO::kVec;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int64_t c = (int64_t(k) * LANES + lane) * V;
        if (c < cols) st16<NT>(reinterpret_cast<u32x4*>(yr + c * IO::kBytes), IO::pack(&v[k * V]));
    }
}

// How a row fits its shape (a template argument of the row kernels):
// kFitAny  any width, any alignment (masks per value where needed);
// kFitVec  width a multiple of the vector on the vector layout (masks per
//          vector, row-independent);
// kFitFull width equal to the shape's capacity on the vector layout (no
//          masks compiled).
constexpr int kFitAny = 0, kFitVec = 1, kFitFull = 2;

// Workgroup size of the single-pass kernels: whole rows, 256 lanes when a
// row takes fewer (several rows per workgroup), else one row.
template <int WPR>
constexpr int reg_threads() {
    return (WPR * kWave >= 256 ? 1 : 256 / (WPR * kWave)) * WPR * kWave;
}

// ------------------------------------------------- single-pass kernel -----
// FIT: what the launcher guarantees about the width (kFitAny, kFitVec,
// kFitFull). Full rows compile no masking code (the masks of ragged rows
// otherwise hold enough SGPRs to cost a wave per SIMD); kFitVec rows mask
// whole vectors (they read as -inf, whose numerators are 0).
template <class IO, int WPR, int VPL, bool VEC, bool NT = false, int FIT = kFitAny>
__global__ __launch_bounds__(reg_threads<WPR>()) void softmax_reg_kernel(
    const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy) {
    constexpr int V = IO::kVec;
    constexpr int E = VPL * V;
    constexpr int kRowLanes = WPR * kWave;
    constexpr int kRowsPerWg = reg_threads<WPR>() / kRowLanes;
    static_assert(FIT == kFitAny || VEC, "fitted rows are a vector-layout case");
    // the column count as the masked helpers see it (a constant for full rows)
    const int64_t span_cols = FIT == kFitFull ? int64_t(kRowLanes) * E : cols;
    // per-wave partials of the row max ([0]) and sum ([1]); one barrier per
    // reduction: a slot is rewritten only on the next row, after every wave
    // has passed the other reduction's barrier, i.e. finished reading it
    __shared__ float red[2][kRowsPerWg * WPR];

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
            if constexpr (FIT == kFitVec)
                load_span_vfit<IO, VPL, kRowLanes, NT>(row_ptr<IO>(x, row, ldx), cols, lr, v,
                                                       kNegInf);
            else
                load_span<IO, VPL, kRowLanes, VEC, NT>(row_ptr<IO>(x, row, ldx), span_cols, 0, lr,
                                                      v);
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
            if (lane == 0) red[0][sub * WPR + wave] = m;
            __syncthreads();
            m = red[0][sub * WPR];
#pragma unroll
            for (int w = 1; w < WPR; ++w) m = fmaxf(m, red[0][sub * WPR + w]);
        }

        // numerators and their sum (masked columns give 2^-inf = 0)
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < E; ++i) {
            v[i] = softmax_numerator(v[i], m);
            s += v[i];
        }
        s = wave_sum(s);
        if constexpr (WPR > 1) {
            if (lane == 0) red[1][sub * WPR + wave] = s;
            __syncthreads();
            s = red[1][sub * WPR];
#pragma unroll
            for (int w = 1; w < WPR; ++w) s += red[1][sub * WPR + w];
        }

        // normalise and write back
        const float r = 1.0f / s;
#pragma unroll
        for (int i = 0; i < E; ++i) v[i] *= r;
        if (active) {
            if constexpr (FIT == kFitVec)
                store_span_vfit<IO, VPL, kRowLanes, NT>(row_ptr<IO>(y, row, ldy), cols, lr, v);
            else
                store_span<IO, VPL, kRowLanes, VEC, NT>(row_ptr<IO>(y, row, ldy), span_cols, 0, lr,
                                                       v);
        }
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

        // pass 1: running (m, l) per lane; l sums unbiased 2^((x - m) log2e)
        float m = kNegInf, l = 0.0f;
        for (int64_t c = 0; c < nchunks; ++c) {
            float v[E];
            load_span<IO, VPL, THREADS, VEC>(xr, cols, c * kChunk, tid, v);
            float cm = kNegInf;
#pragma unroll
            for (int i = 0; i < E; ++i) cm = fmaxf(cm, v[i]);
            const float mn = fmaxf(m, cm);
            if (mn != kNegInf) {  // while every value seen is -inf, l stays 0
                if (mn != m) l *= exp2_raw((m - mn) * kLog2e);
                m = mn;
#pragma unroll
                for (int i = 0; i < E; ++i) l += exp2_raw((v[i] - m) * kLog2e);
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

        // pass 2: normalise, last chunk first; e' carries the factor 2^8
        const float r = 1.0f / (l * kSoftmaxScale);
        for (int64_t c = nchunks - 1; c >= 0; --c) {
            float v[E];
            load_span<IO, VPL, THREADS, VEC>(xr, cols, c * kChunk, tid, v);
#pragma unroll
            for (int i = 0; i < E; ++i) v[i] = softmax_numerator(v[i], m) * r;
            store_span<IO, VPL, THREADS, VEC>(yr, cols, c * kChunk, tid, v);
        }
    }
}

// ------------------------------------------------------------ split kernel -
// Rows wider than one workgroup's registers, without re-reading HBM: the row
// is cut into `parts` slices of THREADS*E columns, one workgroup per slice
// (block b -> row b / parts, slice b % parts), each holding its slice in
// VGPRs. A workgroup reduces its slice to a partial (m_p, l_p) -- the slice
// max and the sum of 2^((x - m_p) log2e) -- publishes it, gathers the row's
// other partials and merges all of them in slice order with the online
// softmax rule ("Lecture 6: GPU Kernels and Triton", section 7.2: the larger
// max wins, the other sum is rescaled by exp(m_old - m_new)). Every slice
// of the row merges the same values in the same order, so all of them
// normalise with bit-identical (M, L).
//
// Exchange: slot[row * parts + p] is one 64-bit word holding (m_p, l_p),
// written and polled with relaxed device-scope atomics. Zero marks an empty
// slot; no real partial is all-zero bits (a finite m_p implies l_p >= 1).
// depart[row] counts the slices that are done with the slots; the last one
// clears the row's slots and its counter, so the workspace is all zero again
// when the kernel ends (it must be all zero before the first call).
//
// The wait for the other slices is bounded by spin_limit polls. Slices of a
// row are consecutive blocks, and blocks are dispatched in order, so the
// wait normally ends within one slice's load time. If the bound is reached,
// the workgroup computes (M, L) by streaming the whole row itself (online
// recurrence) and still normalises its own slice: correct and terminating
// whatever the scheduling, at the cost of that row's bits possibly
// differing in the last place between slices.
constexpr int kSplitMaxParts = kWave;  // one lane polls one slot

__device__ inline unsigned long long pack_ml(float m, float l) {
    return (static_cast<unsigned long long>(__float_as_uint(l)) << 32) | __float_as_uint(m);
}
__device__ inline float unpack_m(unsigned long long w) { return __uint_as_float(uint32_t(w)); }
__device__ inline float unpack_l(unsigned long long w) { return __uint_as_float(uint32_t(w >> 32)); }

// Block-wide max and sum over all THREADS lanes, fixed order, same bits in
// every lane. `red` holds THREADS / 64 floats.
template <int THREADS>
__device__ inline float block_max(float v, float* red) {
    constexpr int kWaves = THREADS / kWave;
    v = wave_max(v);
    if constexpr (kWaves > 1) {
        if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
        __syncthreads();
        v = red[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) v = fmaxf(v, red[w]);
        __syncthreads();
    }
    return v;
}
template <int THREADS>
__device__ inline float block_sum(float v, float* red) {
    constexpr int kWaves = THREADS / kWave;
    v = wave_sum(v);
    if constexpr (kWaves > 1) {
        if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
        __syncthreads();
        v = red[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) v += red[w];
        __syncthreads();
    }
    return v;
}

// (M, L) of a whole row by streaming it once with the online recurrence
// (the fallback of the split kernel). Same bits in every lane.
template <class IO, int THREADS, int VPL, bool VEC>
__device__ inline void row_stats_streamed(const char* xr, int64_t cols, float* red_m,
                                          float* red_l, float& M, float& L) {
    constexpr int E = VPL * IO::kVec;
    constexpr int64_t kChunk = int64_t(THREADS) * E;
    constexpr int kWaves = THREADS / kWave;
    float m = kNegInf, l = 0.0f;
    for (int64_t c0 = 0; c0 < cols; c0 += kChunk) {
        float v[E];
        load_span<IO, VPL, THREADS, VEC>(xr, cols, c0, threadIdx.x, v);
        float cm = kNegInf;
#pragma unroll
        for (int i = 0; i < E; ++i) cm = fmaxf(cm, v[i]);
        const float mn = fmaxf(m, cm);
        if (mn != kNegInf) {
            if (mn != m) l *= exp2_raw((m - mn) * kLog2e);
            m = mn;
#pragma unroll
            for (int i = 0; i < E; ++i) l += exp2_raw((v[i] - m) * kLog2e);
        }
    }
    wave_ml(m, l);
    if (threadIdx.x % kWave == 0) {
        red_m[threadIdx.x / kWave] = m;
        red_l[threadIdx.x / kWave] = l;
    }
    __syncthreads();
    M = red_m[0];
    L = red_l[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) ml_merge(M, L, red_m[w], red_l[w]);
    __syncthreads();
}

template <class IO, int THREADS, int VPL, bool VEC, bool NT = false>
__global__ __launch_bounds__(THREADS) void softmax_split_kernel(
    const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy, int parts,
    unsigned long long* slots, unsigned int* depart, int64_t spin_limit) {
    constexpr int E = VPL * IO::kVec;
    constexpr int64_t kW = int64_t(THREADS) * E;
    constexpr int kWaves = THREADS / kWave;
    __shared__ float red_m[kWaves];
    __shared__ float red_l[kWaves];
    __shared__ float merged[3];  // M, L, gathered-flag

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    // exactly one block per slice (never grid-strided: a block must not wait
    // for a slice queued behind itself)
    const int64_t b = blockIdx.x;
    if (b < rows * parts) {
        const int64_t row = b / parts;
        const int p = static_cast<int>(b - row * parts);
        const char* xr = row_ptr<IO>(x, row, ldx);
        const int64_t c0 = int64_t(p) * kW;

        float v[E];
        load_span<IO, VPL, THREADS, VEC, NT>(xr, cols, c0, tid, v);

        // this slice's partial (m_p, l_p)
        float m = kNegInf;
#pragma unroll
        for (int i = 0; i < E; ++i) m = fmaxf(m, v[i]);
        m = block_max<THREADS>(m, red_m);
        float l = 0.0f;
        if (m != kNegInf) {
#pragma unroll
            for (int i = 0; i < E; ++i) l += exp2_raw((v[i] - m) * kLog2e);
        }
        l = block_sum<THREADS>(l, red_l);

        unsigned long long* row_slots = slots + row * parts;
        if (tid == 0)
            __hip_atomic_store(row_slots + p, pack_ml(m, l), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);

        // wave 0 gathers every slice's partial and merges them in slice order
        if (tid < kWave) {
            unsigned long long w = 0;
            bool gathered = false;
            for (int64_t it = 0;; ++it) {
                w = lane < parts ? __hip_atomic_load(row_slots + lane, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                                 : pack_ml(kNegInf, 0.0f);
                if (__builtin_amdgcn_ballot_w64(w == 0) == 0) {
                    gathered = true;
                    break;
                }
                if (it >= spin_limit) break;
                __builtin_amdgcn_s_sleep(2);
            }
            float pm = unpack_m(w), pl = unpack_l(w);
            wave_ml(pm, pl);
            if (tid == 0) {
                merged[0] = pm;
                merged[1] = pl;
                merged[2] = gathered ? 1.0f : 0.0f;
            }
        }
        __syncthreads();
        float M = merged[0], L = merged[1];
        const bool gathered = merged[2] != 0.0f;
        __syncthreads();
        if (!gathered) row_stats_streamed<IO, THREADS, VPL, VEC>(xr, cols, red_m, red_l, M, L);

        // normalise the slice held in registers
        const float r = 1.0f / (L * kSoftmaxScale);
#pragma unroll
        for (int i = 0; i < E; ++i) v[i] = softmax_numerator(v[i], M) * r;
        store_span<IO, VPL, THREADS, VEC, NT>(row_ptr<IO>(y, row, ldy), cols, c0, tid, v);

        // the last slice done with the row's slots clears them
        if (tid == 0) {
            const unsigned int done =
                __hip_atomic_fetch_add(depart + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (done == static_cast<unsigned int>(parts - 1)) {
                for (int q = 0; q < parts; ++q)
                    __hip_atomic_store(row_slots + q, 0ull, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(depart + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

}  // namespace fk
