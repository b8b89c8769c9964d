// gemm_kernels.hpp -- Linear layer with a fused GELU epilogue on the gfx950
// matrix cores: Y = GELU(X W^T + b), X [M, K], W [N, K] (a Linear weight:
// one row per output feature), b [N], Y [M, N], bf16 or fp16 in and out,
// fp32 accumulation.
//
// This is the Linear -> GELU part of the LayerNorm -> Linear -> GELU fusion
// example of "Lecture 6: GPU Kernels and Triton", section 6.1: the product
// is a dense contraction (compute-bound, section 5), so it runs on MFMA, and
// the activation is applied to the accumulators in registers instead of a
// second kernel that would read and write the M x N product again. The
// tiling follows the same idea as that page's blocked matmul (section 5.1:
// tiles of the output, a K loop over tiles of the operands staged on chip,
// an fp32 accumulator), built here for 64-wide waves and MFMA tiles.
//
// Block tile BM x BN, K step BK; the block's waves form a (BM/WM) x (BN/WN)
// grid, each computing a WM x WN tile as (WM/32) x (WN/32) MFMA 32x32x16
// tiles; the registers are budgeted for OCC waves per SIMD. Two main loops:
//  * linear_gelu_kernel (any K that is a multiple of 8): operand tiles are
//    staged through registers into LDS, double-buffered: the global loads of
//    step k+1 are in flight while step k is multiplied, and one barrier per
//    step separates the buffers. LDS rows are padded by 16 bytes so the
//    16-byte fragment reads of 32 consecutive rows do not pile onto the
//    same banks.
//  * linear_gelu_dtl_kernel (K a multiple of 32 or 64): operands go straight
//    from global memory into a ring of LDS stages (described at the kernel).
// Both multiply in the same k order, so their outputs are bitwise equal.
//
// MFMA 32x32x16 bf16 operand layout (checked on the device): lane l supplies
// A row l % 32 and B column l % 32, each at k = (l / 32) * 8 + e for its 8
// values e; accumulator value v of lane l is C[(v / 4) * 8 + (l / 32) * 4 +
// v % 4][l % 32].
#pragma once

#include "device_common.hpp"

namespace fk {

// epilogue activations of the Linear kernels (the codes of the C ABI)
constexpr int kActNone = 0, kActGelu = 1, kActRelu = 2;


template <int BM_, int BN_, int BK_, int WM_, int WN_, int OCC_ = 1>
struct GemmShape {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int kOcc = OCC_;  // waves per SIMD the registers are budgeted for
    static constexpr int kWavesM = BM / WM, kWavesN = BN / WN;
    static constexpr int kThreads = kWavesM * kWavesN * kWave;
    static constexpr int kTM = WM / 32, kTN = WN / 32;
    static constexpr int kStride = BK + 8;           // bf16 per LDS row (16 bytes of padding)
    static constexpr int kChunksPerRow = BK / 8;     // 16-byte chunks per operand row
    static constexpr int kLoadsA = BM * kChunksPerRow / kThreads;
    static constexpr int kLoadsB = BN * kChunksPerRow / kThreads;
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tiles");
    static_assert(BK % 16 == 0, "K step");
    static_assert(BM * kChunksPerRow % kThreads == 0 && BN * kChunksPerRow % kThreads == 0,
                  "every thread loads whole chunks");
};

// Block index -> output tile (tm, tn). Blocks go to the 8 XCDs round-robin
// (block b on XCD b % 8); when the block count divides by 8 the index is
// first remapped so that each XCD works through a contiguous range of the
// ordering below, then tiles are visited in column-strips of kGemmGroup tile
// rows, so the blocks in flight on one XCD share operand tiles in its L2.
constexpr int kGemmGroup = 4;  // measured best of 4, 8, 16, 32 for 8192 x 16384 x 4096
constexpr int kXcds = 8;

__device__ inline void gemm_tile_of(int64_t b, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                    int64_t& tn) {
    const int64_t nb = tiles_m * tiles_n;
    if (nb % kXcds == 0) b = (b % kXcds) * (nb / kXcds) + b / kXcds;
    const int64_t per_group = int64_t(kGemmGroup) * tiles_n;
    const int64_t g = b / per_group;
    const int64_t first = g * kGemmGroup;
    const int64_t rows = tiles_m - first < kGemmGroup ? tiles_m - first : kGemmGroup;
    const int64_t r = b - g * per_group;
    tm = first + r % rows;
    tn = r / rows;
}

template <class S, class EL = MmaBF16>
__global__ __launch_bounds__(S::kThreads) __attribute__((amdgpu_waves_per_eu(S::kOcc, S::kOcc)))
void linear_gelu_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int64_t ldx, int64_t ldw, int64_t ldy, int act) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][S::BM * S::kStride];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][S::BN * S::kStride];

    const int64_t tiles_m = (M + S::BM - 1) / S::BM;
    const int64_t tiles_n = (N + S::BN - 1) / S::BN;
    int64_t tm, tn;
    gemm_tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = tm * S::BM, n0 = tn * S::BN;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int wm = wave / S::kWavesN, wn = wave % S::kWavesN;

    // this thread's 16-byte chunks of the operand tiles (row, k offset); a
    // step whose tiles lie wholly inside X and W (a uniform test: all but the
    // edge tiles) loads without masks, so all loads are in flight together
    const bool inner_mn = m0 + S::BM <= M && n0 + S::BN <= N;
    u32x4 ra[S::kLoadsA], rb[S::kLoadsB];
    auto load_tiles = [&](int64_t k0) {
        if (inner_mn && k0 + S::BK <= K) {
#pragma unroll
            for (int i = 0; i < S::kLoadsA; ++i) {
                const int c = tid + i * S::kThreads;
                ra[i] = *reinterpret_cast<const u32x4*>(X + (m0 + c / S::kChunksPerRow) * ldx + k0 +
                                                        (c % S::kChunksPerRow) * 8);
            }
#pragma unroll
            for (int i = 0; i < S::kLoadsB; ++i) {
                const int c = tid + i * S::kThreads;
                rb[i] = *reinterpret_cast<const u32x4*>(W + (n0 + c / S::kChunksPerRow) * ldw + k0 +
                                                        (c % S::kChunksPerRow) * 8);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < S::kLoadsA; ++i) {
            const int c = tid + i * S::kThreads;
            const int64_t row = m0 + c / S::kChunksPerRow;
            const int64_t k = k0 + (c % S::kChunksPerRow) * 8;
            ra[i] = (row < M && k < K) ? *reinterpret_cast<const u32x4*>(X + row * ldx + k)
                                       : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < S::kLoadsB; ++i) {
            const int c = tid + i * S::kThreads;
            const int64_t row = n0 + c / S::kChunksPerRow;
            const int64_t k = k0 + (c % S::kChunksPerRow) * 8;
            rb[i] = (row < N && k < K) ? *reinterpret_cast<const u32x4*>(W + row * ldw + k)
                                       : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int i = 0; i < S::kLoadsA; ++i) {
            const int c = tid + i * S::kThreads;
            *reinterpret_cast<u32x4*>(&As[buf][(c / S::kChunksPerRow) * S::kStride +
                                               (c % S::kChunksPerRow) * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < S::kLoadsB; ++i) {
            const int c = tid + i * S::kThreads;
            *reinterpret_cast<u32x4*>(&Bs[buf][(c / S::kChunksPerRow) * S::kStride +
                                               (c % S::kChunksPerRow) * 8]) = rb[i];
        }
    };

    f32x16 acc[S::kTM][S::kTN];
#pragma unroll
    for (int i = 0; i < S::kTM; ++i)
#pragma unroll
        for (int j = 0; j < S::kTN; ++j) acc[i][j] = f32x16{};

    const int64_t nk = (K + S::BK - 1) / S::BK;
    load_tiles(0);
    store_tiles(0);
    __syncthreads();
    const int frag_row = lane % 32;
    const int frag_k = (lane / 32) * 8;
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int buf = static_cast<int>(kt & 1);
        if (kt + 1 < nk) load_tiles((kt + 1) * S::BK);
        const uint16_t* a_base = &As[buf][(wm * S::WM + frag_row) * S::kStride + frag_k];
        const uint16_t* b_base = &Bs[buf][(wn * S::WN + frag_row) * S::kStride + frag_k];
#pragma unroll
        for (int kk = 0; kk < S::BK / 16; ++kk) {
            typename EL::frag af[S::kTM], bf[S::kTN];
#pragma unroll
            for (int i = 0; i < S::kTM; ++i)
                af[i] = *reinterpret_cast<const typename EL::frag*>(a_base + i * 32 * S::kStride + kk * 16);
#pragma unroll
            for (int j = 0; j < S::kTN; ++j)
                bf[j] = *reinterpret_cast<const typename EL::frag*>(b_base + j * 32 * S::kStride + kk * 16);
#pragma unroll
            for (int i = 0; i < S::kTM; ++i)
#pragma unroll
                for (int j = 0; j < S::kTN; ++j)
                    acc[i][j] = EL::mfma(af[i], bf[j], acc[i][j]);
        }
        if (kt + 1 < nk) store_tiles(buf ^ 1);
        __syncthreads();
    }

    // epilogue: + bias, the activation on the accumulators, round, store
#pragma unroll
    for (int j = 0; j < S::kTN; ++j) {
        const int64_t col = n0 + wn * S::WN + j * 32 + lane % 32;
        const float bv = (bias != nullptr && col < N) ? EL::load1(bias, col) : 0.0f;
#pragma unroll
        for (int i = 0; i < S::kTM; ++i) {
            float v[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = acc[i][j][e] + bv;
            if (act == kActGelu) {
                gelu_tanh_n(v);
            } else if (act == kActRelu) {
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] = relu1(v[e]);
            }
            const int64_t row0 = m0 + wm * S::WM + i * 32 + (lane / 32) * 4;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = row0 + (e / 4) * 8 + e % 4;
                if (row < M && col < N) EL::store1(Y, row * ldy + col, v[e]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Main loop fed by direct global -> LDS loads (global_load_lds_dwordx4: lane
// i of a wave writes its 16 bytes at LDS base + 16 i, no registers and no
// LDS store instructions). Operand tiles go through a ring of kStages LDS
// stages, loaded kStages - 1 K steps ahead; each step waits for its own
// stage with a counted wait on the loads still in flight, then one barrier.
//
// LDS layout of a stage: A rows then B rows, each row BK bf16 = BK / 8
// chunks of 16 bytes, chunk c of row r stored at chunk position c ^ swz(r):
// (r >> 2) & 3 for 64-byte rows (BK 32), (r >> 1) & 7 for 128-byte rows
// (BK 64). The MFMA fragment reads (16 consecutive rows, one chunk, per
// quarter wave) then spread over all 16 bank groups of 16 bytes. A wave's
// direct load fills 1 KiB, 1024 / (2 BK) rows, so lane i fetches row
// i / (BK / 8), chunk (i % (BK / 8)) ^ swz(row).
//
// K steps of 64 when K allows: a load then covers whole 128-byte lines (8
// rows), where K steps of 32 request half lines (16 rows of 64 bytes), twice
// the requests to L2 for the same bytes; with two stages of 64 KiB each K
// step's loads have the previous step to land (8192 x 16384 x 4096: 1.031
// -> 0.992 ms, bitwise the same outputs: same k order).
//
// Rows past M or N load row M - 1 or N - 1 instead (valid memory; those
// outputs are never stored). K must be a multiple of BK.
template <int BM_, int BN_, int WM_, int WN_, int OCC_, int STAGES_, int BK_ = 32>
struct DtlShape {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int kOcc = OCC_, kStages = STAGES_;
    static constexpr int kWavesM = BM / WM, kWavesN = BN / WN;
    static constexpr int kWaves = kWavesM * kWavesN;
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int kTM = WM / 32, kTN = WN / 32;
    static constexpr int kRowBytes = BK * 2;                      // 64 or 128
    static constexpr int kChunks = BK / 8;                        // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;         // rows of one 1 KiB wave load
    static constexpr int kStageBytes = (BM + BN) * kRowBytes;
    static constexpr int kLoadsPerWave = (BM + BN) / kRowsPerLoad / kWaves;  // per step
    static_assert(BK == 32 || BK == 64, "K steps of 32 or 64");
    static_assert((BM + BN) % (kRowsPerLoad * kWaves) == 0, "whole wave loads");
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tiles");
    static_assert(kStages >= 2 && kStages * kStageBytes <= 160 * 1024, "LDS");
    // chunk position of logical chunk c of stage row r: c ^ swz(r)
    __device__ static constexpr int swz(int r) { return BK == 32 ? ((r >> 2) & 3) : ((r >> 1) & 7); }
};

typedef __attribute__((address_space(3))) void* las_ptr;

// One direct 16-byte load per lane into LDS at lds_base + 16 * lane. Issued
// from inline assembly so that the compiler does not track it: its own
// tracking of such loads waits for all of them (vmcnt(0)) before every
// barrier and every LDS read, which would serialise the stage ring. The
// kernel waits for them itself (vmcnt_imm); "memory" keeps the compiler from
// moving LDS reads across the statement or treating the LDS as unwritten.
// M0 is a register the compiler reserves; it warns that a clobber of it is
// not saved. Nothing else in these kernels uses M0 (gfx9 LDS instructions do
// not), so it is only ever set here, right before the load that reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void lds_dma16(const void* gsrc, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gsrc), "s"(lds_base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate waiting for at most n outstanding vector memory
// operations (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima, i.e. not waited for)
__device__ constexpr int vmcnt_imm(int n) {
    return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

template <class S, class EL = MmaBF16>
__global__ __launch_bounds__(S::kThreads) __attribute__((amdgpu_waves_per_eu(S::kOcc, S::kOcc)))
void linear_gelu_dtl_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                            const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
                            int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                            int act) {
    __shared__ __attribute__((aligned(1024))) char smem[S::kStages * S::kStageBytes];

    const int64_t tiles_m = (M + S::BM - 1) / S::BM;
    const int64_t tiles_n = (N + S::BN - 1) / S::BN;
    int64_t tm, tn;
    gemm_tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = tm * S::BM, n0 = tn * S::BN;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int wm = wave / S::kWavesN, wn = wave % S::kWavesN;

    // this lane's source rows for its wave's loads (row groups of
    // kRowsPerLoad of the stage: A rows 0 .. BM - 1, then B rows), with the
    // chunk swizzle
    const int lrow = lane / S::kChunks;
    const int lpos = lane % S::kChunks;
    const uint16_t* src[S::kLoadsPerWave];
#pragma unroll
    for (int j = 0; j < S::kLoadsPerWave; ++j) {
        const int grp = wave * S::kLoadsPerWave + j;  // row group of the stage
        const int r = grp * S::kRowsPerLoad + lrow;
        const int lchunk = lpos ^ S::swz(r);
        if (r < S::BM) {
            const int64_t row = m0 + r < M ? m0 + r : M - 1;
            src[j] = X + row * ldx + lchunk * 8;
        } else {
            const int64_t row = n0 + (r - S::BM) < N ? n0 + (r - S::BM) : N - 1;
            src[j] = W + row * ldw + lchunk * 8;
        }
    }
    auto issue = [&](int kt) {  // loads of K step kt into stage kt % kStages
        char* stage = smem + (kt % S::kStages) * S::kStageBytes;
#pragma unroll
        for (int j = 0; j < S::kLoadsPerWave; ++j) {
            const int grp = wave * S::kLoadsPerWave + j;
            // LDS byte address of the wave's 1 KiB (wave-uniform: an SGPR)
            const uint32_t dst = __builtin_amdgcn_readfirstlane(
                static_cast<uint32_t>(reinterpret_cast<uintptr_t>((las_ptr)(stage + grp * 1024))));
            lds_dma16(src[j] + kt * S::BK, dst);
        }
    };

    f32x16 acc[S::kTM][S::kTN];
#pragma unroll
    for (int i = 0; i < S::kTM; ++i)
#pragma unroll
        for (int j = 0; j < S::kTN; ++j) acc[i][j] = f32x16{};

    // 32-bit step counters (the host refuses K >= 2^36), and what only the
    // epilogue needs (M, N, ldy, the bias and output pointers) carried across
    // the main loop as lane values (an empty asm makes them opaque): 64-bit
    // step counters and those scalars kept live through the loop filled the
    // SGPR budget, and the compiler spilled 24 SGPRs to VGPR lanes
    const int nk = static_cast<int>(K / S::BK);
    int64_t Mv = M, Nv = N, ldyv = ldy;
    const uint16_t* biasv = bias;
    uint16_t* Yv = Y;
    asm volatile("" : "+v"(Mv), "+v"(Nv), "+v"(ldyv), "+v"(biasv), "+v"(Yv));
#pragma unroll
    for (int st = 0; st < S::kStages - 1; ++st)
        if (st < nk) issue(st);

    // fragment rows of this lane and the swizzled chunk offsets per kk
    const int frow = lane % 32;
    for (int kt = 0; kt < nk; ++kt) {
        // stage kt landed: at most (kStages - 2) later steps' loads in flight
        if (kt + S::kStages - 2 < nk)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((S::kStages - 2) * S::kLoadsPerWave));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();  // every wave's part of stage kt; stage kt - 1 free
        if (kt + S::kStages - 1 < nk) issue(kt + S::kStages - 1);

        const char* stage = smem + (kt % S::kStages) * S::kStageBytes;
#pragma unroll
        for (int kk = 0; kk < S::BK / 16; ++kk) {
            const int c = kk * 2 + lane / 32;  // logical chunk of this lane's 8 k values
            typename EL::frag af[S::kTM], bf[S::kTN];
#pragma unroll
            for (int i = 0; i < S::kTM; ++i) {
                const int r = wm * S::WM + i * 32 + frow;
                af[i] = *reinterpret_cast<const typename EL::frag*>(stage + r * S::kRowBytes +
                                                         ((c ^ S::swz(r)) << 4));
            }
#pragma unroll
            for (int j = 0; j < S::kTN; ++j) {
                const int r = S::BM + wn * S::WN + j * 32 + frow;
                bf[j] = *reinterpret_cast<const typename EL::frag*>(stage + r * S::kRowBytes +
                                                         ((c ^ S::swz(r)) << 4));
            }
#pragma unroll
            for (int i = 0; i < S::kTM; ++i)
#pragma unroll
                for (int j = 0; j < S::kTN; ++j)
                    acc[i][j] = EL::mfma(af[i], bf[j], acc[i][j]);
        }
    }

    // epilogue: + bias, the activation on the accumulators, round, store
    const int64_t ldy5 = 5 * ldyv;
#pragma unroll
    for (int j = 0; j < S::kTN; ++j) {
        const int64_t col = n0 + wn * S::WN + j * 32 + lane % 32;
        const float bv = (biasv != nullptr && col < Nv) ? EL::load1(biasv, col) : 0.0f;
#pragma unroll
        for (int i = 0; i < S::kTM; ++i) {
            float v[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = acc[i][j][e] + bv;
            if (act == kActGelu) {
                gelu_tanh_n(v);
            } else if (act == kActRelu) {
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] = relu1(v[e]);
            }
            // rows row0 + (e / 4) * 8 + e % 4, reached by stepping one
            // pointer (scalar strides) rather than by 16 row products, whose
            // 64-bit scalars would spill the SGPRs
            const int64_t row0 = m0 + wm * S::WM + i * 32 + (lane / 32) * 4;
            const int64_t left = Mv - row0;
            uint16_t* p = Yv + row0 * ldyv + col;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if ((e / 4) * 8 + e % 4 < left && col < Nv) EL::store1(p, 0, v[e]);
                p += (e % 4 == 3) ? ldy5 : ldyv;
            }
        }
    }
}

}  // namespace fk
