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

// ---------------------------------------------------------- staged kernel -
// The online two-pass kernel for 16-byte-aligned rows, keeping as much of the
// row on chip as a 512-lane workgroup can hold, so that only the rest is
// read from HBM twice. The row is cut into chunks of THREADS * VPL 16-byte
// vectors (one vector per lane per k < VPL, the layout of load_span); chunk
// c < RREG stays in the lanes' VGPRs as raw 16-byte words, chunk
// RREG <= c < RREG + RLDS in LDS, and the chunks after those are streamed.
// Pass 1 updates a per-lane running max m and sum l chunk by chunk: when the
// max grows, l is rescaled by 2^((m_old - m_new) log2e) ("Lecture 6: GPU
// Kernels and Triton", section 7.2 "Online Softmax", without the attention
// accumulator); the lanes' states then merge by the same rule (wave by DPP,
// waves through LDS, a fixed order). Pass 2 normalises: the streamed chunks
// are read again (last first: the most recently read bytes are the likeliest
// to be in L2 or the Infinity Cache), the resident ones come from VGPRs and
// LDS. Each resident element is read from HBM once and written once.
//
// With the launcher's shapes (8192-column chunks, two waves per SIMD at 256
// VGPRs; fp32: VPL 4, RREG 12, RLDS 4; bf16: VPL 2, RREG 24, RLDS 8) the
// first 131072 fp32 or 262144 bf16 columns (512 KiB) stay on chip: a
// 1024 x 131072 fp32 row is read from HBM once.
template <class IO, int VPL, int LANES, bool NT>
__device__ inline void load_raw_span(const char* xr, int64_t cols, int64_t c0, int lane,
                                     u32x4 (&w)[VPL]) {
    constexpr int V = IO::kVec;
    constexpr int64_t kSpan = int64_t(VPL) * LANES * V;
    if (cols - c0 >= kSpan) {
#pragma unroll
        for (int k = 0; k < VPL; ++k)
            w[k] = ld16<NT>(reinterpret_cast<const u32x4*>(
                xr + (c0 + (int64_t(k) * LANES + lane) * V) * IO::kBytes));
        return;
    }
    // the row's last, partial chunk: whole vectors where they fit, single
    // elements for the one straddling the row end, -inf past it (a bf16 or
    // fp32 value widened and rounded back is itself, -inf included)
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int64_t c = c0 + (int64_t(k) * LANES + lane) * V;
        if (c + V <= cols) {
            w[k] = ld16<NT>(reinterpret_cast<const u32x4*>(xr + c * IO::kBytes));
        } else {
            float v[V];
#pragma unroll
            for (int e = 0; e < V; ++e) v[e] = (c + e < cols) ? IO::load1(xr, c + e) : kNegInf;
            w[k] = IO::pack(v);
        }
    }
}

// Per-lane online update of (m, l) with the values of one chunk.
template <class IO, int VPL>
__device__ inline void ml_update_raw(const u32x4 (&w)[VPL], float& m, float& l) {
    constexpr int E = VPL * IO::kVec;
    float v[E];
#pragma unroll
    for (int k = 0; k < VPL; ++k) IO::unpack(w[k], &v[k * IO::kVec]);
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

// y for one chunk from its raw words: e' / (l 2^8), stored (masked past cols).
template <class IO, int VPL, int LANES, bool NT>
__device__ inline void normalise_store_raw(char* yr, int64_t cols, int64_t c0, int lane,
                                           const u32x4 (&w)[VPL], float M, float r) {
    constexpr int E = VPL * IO::kVec;
    float v[E];
#pragma unroll
    for (int k = 0; k < VPL; ++k) IO::unpack(w[k], &v[k * IO::kVec]);
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = softmax_numerator(v[i], M) * r;
    store_span<IO, VPL, LANES, true, NT>(yr, cols, c0, lane, v);
}

// Resident chunks are loaded with buffer instructions: the row is one buffer
// resource (scalar registers), every load of a lane shares one VGPR offset
// (tid * 16) and adds a scalar offset per chunk and vector. Global loads
// would need a 64-bit VGPR address each (the strides between a lane's
// vectors exceed their immediate offsets), which the compiler computes ahead
// and keeps live: that spilled. Rows of < 2^31 bytes only (32-bit offsets).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Word 3 of a raw buffer descriptor on this architecture family: data
// format 32 bits (a zero format would make every access return 0).
constexpr int kBufferWord3 = 0x00020000;

__device__ inline rsrc_t row_buffer(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             kBufferWord3);
}

// The VPL vectors of a lane in chunk c (a whole chunk: no masks). voff is
// the lane's byte offset (tid * 16), chunk_bytes the chunk size in bytes.
template <int VPL, int LANES, bool NT>
__device__ inline void load_chunk_buf(rsrc_t rx, uint32_t voff, uint32_t c0_bytes,
                                      u32x4 (&w)[VPL]) {
#pragma unroll
    for (int k = 0; k < VPL; ++k)
        w[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, voff, c0_bytes + k * LANES * 16, NT ? 2 : 0);
}

// The same chunk straight into LDS (buffer_load_dwordx4 ... lds, no VGPRs):
// for vector k, wave w's 64 lanes write 16 bytes each, in lane order, at
// &dst[k][w * 64], so lane tid's vector lands at dst[k][tid].
template <int VPL, int LANES, bool NT>
__device__ inline void load_chunk_lds(rsrc_t rx, uint32_t voff, uint32_t c0_bytes, int tid,
                                      u32x4 (*dst)[LANES]) {
    const int wave_base = (tid / kWave) * kWave;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (__attribute__((address_space(3))) void*)(&dst[k][wave_base]), 16, voff,
            c0_bytes + k * LANES * 16, 0, NT ? 2 : 0);
}

// y for one whole chunk, stored with global instructions from the row base
// plus a 32-bit lane offset. (Buffer stores were tried here: in 512-lane
// workgroups storing eight or more chunks per lane, lanes 12-15 of every
// 16-lane group in waves 4-7 stored values that the next instruction had
// already written into the store's data registers; global stores are
// exact in the same kernel.)
template <class IO, int VPL, int LANES, bool NT>
__device__ inline void normalise_store_global(char* yr, uint32_t voff, uint32_t c0_bytes,
                                              const u32x4 (&w)[VPL], float M, float r) {
    constexpr int V = IO::kVec;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        float v[V];
        IO::unpack(w[k], v);
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = softmax_numerator(v[e], M) * r;
        const uint32_t off = c0_bytes + k * LANES * 16 + voff;
        st16<NT>(reinterpret_cast<u32x4*>(yr + off), IO::pack(v));
    }
}

// The lane index as an opaque value: everything computed from it after this
// point stays after it. The masked chunk path derives per-lane columns and
// 64-bit compares from the lane alone; left visible, the compiler hoists them
// out of the row loop and keeps them live beside the resident chunks, which
// then spill.
__device__ inline int opaque_lane(int tid) {
    asm volatile("" : "+v"(tid));
    return tid;
}

template <class IO, int THREADS, int VPL, int RREG, int RLDS, bool NT>
__global__ __launch_bounds__(THREADS) void softmax_staged_kernel(
    const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy) {
    constexpr int64_t kChunk = int64_t(THREADS) * VPL * IO::kVec;
    constexpr int kWaves = THREADS / kWave;
    // LDS chunks as raw words, [chunk][vector k][lane]: a lane's 16 bytes of
    // one k are contiguous with its neighbours' (conflict-free 128-bit access)
    __shared__ u32x4 stage[RLDS > 0 ? RLDS : 1][VPL][THREADS];
    __shared__ float red_m[kWaves];
    __shared__ float red_l[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int64_t nchunks = (cols + kChunk - 1) / kChunk;
    const int64_t nfull = cols / kChunk;
    // chunks from here on are streamed (read in both passes)
    const int64_t first_streamed = nfull < RREG + RLDS ? nfull : RREG + RLDS;
    const bool streams = first_streamed < nchunks;

    constexpr uint32_t kChunkBytes = uint32_t(kChunk) * IO::kBytes;
    const uint32_t voff = uint32_t(tid) * 16;
    const uint32_t row_bytes = uint32_t(cols) * IO::kBytes;

    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const char* xr = row_ptr<IO>(x, row, ldx);
        char* yr = row_ptr<IO>(y, row, ldy);
        const rsrc_t rx = row_buffer(xr, row_bytes);

        // pass 1: every load in flight first
        u32x4 res[RREG][VPL];
#pragma unroll
        for (int c = 0; c < RREG; ++c)
            if (c < nfull) load_chunk_buf<VPL, THREADS, NT>(rx, voff, c * kChunkBytes, res[c]);
#pragma unroll
        for (int c = RREG; c < RREG + RLDS; ++c)
            if (c < nfull)
                load_chunk_lds<VPL, THREADS, NT>(rx, voff, c * kChunkBytes, tid, stage[c - RREG]);
        u32x4 t[VPL];
        if (streams) load_raw_span<IO, VPL, THREADS, NT>(xr, cols, first_streamed * kChunk, opaque_lane(tid), t);

        float m = kNegInf, l = 0.0f;
#pragma unroll
        for (int c = 0; c < RREG; ++c)
            if (c < nfull) ml_update_raw<IO, VPL>(res[c], m, l);
        // the LDS chunks: each lane reads back what its own loads wrote, once
        // they have completed
        __builtin_amdgcn_s_waitcnt(0);
        // (one LDS chunk at a time: the scheduler would otherwise hoist
        // every chunk's reads together, and the registers they need spill)
#pragma unroll
        for (int c = RREG; c < RREG + RLDS; ++c) {
            if (c < nfull) {
                u32x4 w[VPL];
#pragma unroll
                for (int k = 0; k < VPL; ++k) w[k] = stage[c - RREG][k][tid];
                ml_update_raw<IO, VPL>(w, m, l);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (streams) ml_update_raw<IO, VPL>(t, m, l);
        for (int64_t c = first_streamed + 1; c < nchunks; ++c) {
            load_raw_span<IO, VPL, THREADS, NT>(xr, cols, c * kChunk, opaque_lane(tid), t);
            ml_update_raw<IO, VPL>(t, m, l);
        }

        // merge the lanes' states: the wave (DPP), then the waves (LDS)
        wave_ml(m, l);
        if (lane == 0) {
            red_m[wave] = m;
            red_l[wave] = l;
        }
        __syncthreads();
        float M = red_m[0], L = red_l[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) ml_merge(M, L, red_m[w], red_l[w]);

        // pass 2: e' carries the factor 2^8. bf16 resident words pass
        // through an empty asm statement first, so the compiler unpacks them
        // again here rather than keeping pass 1's unpacked values alive
        // (twice the registers); fp32 words need no unpacking.
        if constexpr (IO::kBytes == 2) {
#pragma unroll
            for (int c = 0; c < RREG; ++c)
#pragma unroll
                for (int k = 0; k < VPL; ++k) asm volatile("" : "+v"(res[c][k]));
        }
        const float r = 1.0f / (L * kSoftmaxScale);
        if (streams)
            load_raw_span<IO, VPL, THREADS, NT>(xr, cols, (nchunks - 1) * kChunk, opaque_lane(tid), t);
#pragma unroll
        for (int c = 0; c < RREG; ++c)
            if (c < nfull)
                normalise_store_global<IO, VPL, THREADS, NT>(yr, voff, c * kChunkBytes, res[c], M, r);
#pragma unroll
        for (int c = RREG; c < RREG + RLDS; ++c) {
            if (c < nfull) {
                u32x4 w[VPL];
#pragma unroll
                for (int k = 0; k < VPL; ++k) w[k] = stage[c - RREG][k][tid];
                normalise_store_global<IO, VPL, THREADS, NT>(yr, voff, c * kChunkBytes, w, M, r);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (streams) {
            normalise_store_raw<IO, VPL, THREADS, NT>(yr, cols, (nchunks - 1) * kChunk, opaque_lane(tid), t,
                                                      M, r);
            for (int64_t c = nchunks - 2; c >= first_streamed; --c) {
                load_raw_span<IO, VPL, THREADS, NT>(xr, cols, c * kChunk, opaque_lane(tid), t);
                normalise_store_raw<IO, VPL, THREADS, NT>(yr, cols, c * kChunk, opaque_lane(tid), t,
                                                          M, r);
            }
        }
        // the next row rewrites red_m / red_l and the LDS chunks
        __syncthreads();
    }
}

// s_waitcnt immediate: at most n vector memory operations of this wave in
// flight (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at
// their maxima, i.e. not waited for)
__device__ constexpr int vmcnt_count(int n) {
    return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// ---------------------------------------------------------- rolling kernel -
// The staged kernel for rows that stay on chip whole (exactly RREG + RLDS
// chunks), with a persistent grid (at most one workgroup per CU, each
// looping over rows) that overlaps a row's second pass with the next row's
// first: in pass 2, as soon as chunk c of row r is normalised and stored,
// the same registers (or LDS words) take chunk c of the workgroup's next
// row, and chunk c - D of that next row (landed by then: a counted wait
// lets the later D chunks' stores and loads stay in flight) goes into the
// next row's running (m, l). The staged kernel reads a whole row, reduces
// it, then writes it, so the GPU alternates between read-only and
// write-only phases with gaps between them. Each LDS chunk word is written
// and read by the same lane (the direct loads of a wave fill that wave's
// own lanes' slots), so no barrier guards their reuse. Same arithmetic, in
// the same order, as the staged kernel.
template <class IO, int THREADS, int VPL, int RREG, int RLDS, bool NT>
__global__ __launch_bounds__(THREADS) void softmax_rolling_kernel(
    const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy) {
    constexpr int64_t kChunk = int64_t(THREADS) * VPL * IO::kVec;
    constexpr int kWaves = THREADS / kWave;
    constexpr int NC = RREG + RLDS;   // chunks per row (cols == NC * kChunk)
    constexpr int D = 2;              // chunks the next row's pass 1 trails its loads by
    constexpr int kOps = 2 * VPL;     // memory operations per chunk in pass 2
    static_assert(NC > D && D == 2 && D * kOps <= 63, "counted waits");
    __shared__ u32x4 stage[RLDS > 0 ? RLDS : 1][VPL][THREADS];
    __shared__ float red_m[kWaves];
    __shared__ float red_l[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    constexpr uint32_t kChunkBytes = uint32_t(kChunk) * IO::kBytes;
    const uint32_t voff = uint32_t(tid) * 16;
    const uint32_t row_bytes = uint32_t(cols) * IO::kBytes;

    u32x4 res[RREG][VPL];
    // chunk c of the lane's words into (m, l)
    auto update = [&](int c, float& m, float& l) {
        if (c < RREG) {
            ml_update_raw<IO, VPL>(res[c], m, l);
        } else {
            u32x4 w[VPL];
#pragma unroll
            for (int k = 0; k < VPL; ++k) w[k] = stage[c - RREG][k][tid];
            ml_update_raw<IO, VPL>(w, m, l);
        }
    };
    auto load_chunk = [&](rsrc_t rx, int c) {
        if (c < RREG) load_chunk_buf<VPL, THREADS, NT>(rx, voff, c * kChunkBytes, res[c]);
        else load_chunk_lds<VPL, THREADS, NT>(rx, voff, c * kChunkBytes, tid, stage[c - RREG]);
    };

    // the first row: loaded and reduced on its own
    float m = kNegInf, l = 0.0f;
    if (int64_t(blockIdx.x) < rows) {
        const rsrc_t rx = row_buffer(row_ptr<IO>(x, blockIdx.x, ldx), row_bytes);
#pragma unroll
        for (int c = 0; c < NC; ++c) load_chunk(rx, c);
        __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            update(c, m, l);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const int64_t next = row + gridDim.x;
        const bool more = next < rows;
        char* yr = row_ptr<IO>(y, row, ldy);

        // merge the lanes' states of this row: the wave (DPP), then the waves
        wave_ml(m, l);
        if (lane == 0) {
            red_m[wave] = m;
            red_l[wave] = l;
        }
        __syncthreads();
        float M = red_m[0], L = red_l[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) ml_merge(M, L, red_m[w], red_l[w]);

        // pass 2 of this row, the loads and pass 1 of the next
        if constexpr (IO::kBytes == 2) {
#pragma unroll
            for (int c = 0; c < RREG; ++c)
#pragma unroll
                for (int k = 0; k < VPL; ++k) asm volatile("" : "+v"(res[c][k]));
        }
        const float r = 1.0f / (L * kSoftmaxScale);
        const rsrc_t rn = row_buffer(row_ptr<IO>(x, more ? next : row, ldx), row_bytes);
        m = kNegInf;
        l = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (c < RREG) {
                normalise_store_global<IO, VPL, THREADS, NT>(yr, voff, c * kChunkBytes, res[c], M, r);
            } else {
                u32x4 w[VPL];
#pragma unroll
                for (int k = 0; k < VPL; ++k) w[k] = stage[c - RREG][k][tid];
                normalise_store_global<IO, VPL, THREADS, NT>(yr, voff, c * kChunkBytes, w, M, r);
                // this lane's words are read before its wave's direct load
                // replaces them
                __builtin_amdgcn_s_waitcnt(0xC07F);
            }
            if (more) {
                load_chunk(rn, c);
                if (c >= D) {
                    // chunk c - D landed: only the D later chunks' stores and
                    // loads may be in flight
                    __builtin_amdgcn_s_waitcnt(vmcnt_count(D * kOps));
                    update(c - D, m, l);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (more) {  // the last D = 2 chunks of the next row
            __builtin_amdgcn_s_waitcnt(vmcnt_count(kOps));
            update(NC - 2, m, l);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_count(0));
            update(NC - 1, m, l);
        }
        // the next row rewrites red_m / red_l
        __syncthreads();
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
// Exchange: slot p of a row is two 64-bit words, (epoch << 32 | bits of
// m_p) and (epoch << 32 | bits of l_p), written and polled with relaxed
// device-scope atomics. `epoch` is a non-zero tag the host draws afresh for
// every launch; a word counts only when it carries this launch's tag, so
// whatever the workspace held before -- zeros, another call's partials,
// garbage -- is never taken for a partial of this call (a stale word would
// have to match the 32-bit tag in both words). The workspace therefore
// needs no clearing before or after a call.
//
// The wait for the other slices is bounded by spin_limit polls. Slices of a
// row are consecutive blocks, and blocks are dispatched in order, so the
// wait normally ends within one slice's load time. If the bound is reached,
// the workgroup computes (M, L) by streaming the whole row itself (online
// recurrence) and still normalises its own slice: correct and terminating
// whatever the scheduling, at the cost of that row's bits possibly
// differing in the last place between slices. The streamed statistics
// re-read x after other slices of the row may have written y, so the host
// never sends an in-place call (y == x) down this path.
constexpr int kSplitMaxParts = kWave;  // one lane polls one slot

__device__ inline unsigned long long tag_word(uint32_t epoch, float v) {
    return (static_cast<unsigned long long>(epoch) << 32) | __float_as_uint(v);
}
__device__ inline uint32_t word_tag(unsigned long long w) { return uint32_t(w >> 32); }
__device__ inline float word_value(unsigned long long w) { return __uint_as_float(uint32_t(w)); }

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
    unsigned long long* slots, uint32_t epoch, int64_t spin_limit) {
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

        unsigned long long* row_slots = slots + 2 * (row * parts);
        if (tid == 0) {
            __hip_atomic_store(row_slots + 2 * p, tag_word(epoch, m), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(row_slots + 2 * p + 1, tag_word(epoch, l), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }

        // wave 0 gathers every slice's partial and merges them in slice order
        if (tid < kWave) {
            float pm = kNegInf, pl = 0.0f;  // lanes past the slices hold the empty state
            bool gathered = false;
            for (int64_t it = 0;; ++it) {
                bool have = true;
                if (lane < parts) {
                    const unsigned long long wm = __hip_atomic_load(
                        row_slots + 2 * lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const unsigned long long wl = __hip_atomic_load(
                        row_slots + 2 * lane + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    have = word_tag(wm) == epoch && word_tag(wl) == epoch;
                    pm = word_value(wm);
                    pl = word_value(wl);
                }
                if (__builtin_amdgcn_ballot_w64(!have) == 0) {
                    gathered = true;
                    break;
                }
                if (it >= spin_limit) break;
                __builtin_amdgcn_s_sleep(2);
            }
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
    }
}

}  // namespace fk
