// attention_kernels.hpp -- FlashAttention forward for gfx950 (bf16 or fp16
// in and out, fp32 statistics and accumulators, head dimension 128).
//
// O = softmax(Q K^T / sqrt(d) + mask) V, computed tile by tile without
// materialising the T x T scores ("Lecture 6: GPU Kernels and Triton",
// sections 7.3 and 8): for a block of queries, loop over blocks of keys,
// S_ij = Q_i K_j^T / sqrt(d), update the running max m and sum l with the
// online softmax rule (rescale the old sum and accumulator by
// exp(m_old - m_new)), add P_ij V_j to the accumulator, and divide by l at
// the end. As on that page, P is rounded to the input dtype before the
// P V product. The causal mask keeps key j for query i when j <= i.
//
// MI355X mapping. Each wave owns 32 queries; a workgroup of W waves owns
// 32 W queries of one (batch, head) and walks the key blocks of 64 keys,
// staged through LDS (K as [key][dim], V transposed as [dim][key], both
// double-buffered, loaded one block ahead through registers). The wave
// computes the transposed scores S^T = K Q^T with the 32x32x16 bf16 MFMA:
// K is the A operand (lane l: key l % 32, dims (l / 32) * 8 + e), Q the B
// operand (query l % 32), held in registers for the whole key loop. In the
// accumulator layout of S^T every lane holds one query (l % 32) and 16 of
// the 32 keys of a tile (lane l ^ 32 holds the other 16), so the row max and
// sum of a query are a lane-local reduction plus one exchange with lane
// l ^ 32, and the rescaling of the output accumulator is per lane. The P V
// product is computed as O^T = V^T P^T: P^T is the B operand and comes
// straight from the lane's S^T registers (rounded to bf16) -- the MFMA's
// k index g * 8 + e (g = l / 32) is taken to mean key 8 (e / 4) + 4 g + e % 4
// of each 16-key chunk, which is the order the accumulator layout holds
// them in, and V^T's A fragments are read from LDS in the same key order
// (two 8-byte runs). The output accumulator O^T again holds one query per
// lane, so the final division by l is per lane.
#pragma once

#include "device_common.hpp"
#include "gemm_kernels.hpp"

namespace fk {

constexpr int kAttnD = 128;       // head dimension
constexpr int kAttnBC = 64;       // keys per block
constexpr int kAttnWaves = 4;     // waves per workgroup (32 queries each)
constexpr int kAttnThreads = kAttnWaves * kWave;
constexpr int kAttnBQ = kAttnWaves * 32;
constexpr int kKStride = kAttnD + 8;    // bf16 per K row in LDS (16 bytes of padding)
constexpr int kVtStride = kAttnBC + 8;  // bf16 per V^T row in LDS
constexpr int kAttnChunks = kAttnBC * kAttnD / 8;               // 16-byte chunks per block
constexpr int kAttnLoads = kAttnChunks / kAttnThreads;          // per thread, per operand

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    int64_t B, H, T;
    int64_t qb, qh, qt;  // strides in elements (the head dimension is contiguous)
    int64_t kb, kh, kt;
    int64_t vb, vh, vt;
    int64_t ob, oh, ot;
    float scale_log2;  // log2(e) / sqrt(d)
    int causal;
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two waves per SIMD (two workgroups per CU; LDS 70 KiB each): with one, a
// wave's MFMA, exponential and LDS phases run back to back and the K/V loads
// barely overlap them; the second workgroup fills those gaps. The compiler
// fits the kernel in 256 registers (no AGPRs, no spills) when asked to.
template <class EL>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attention_fwd_kernel(AttnArgs a) {  // EL: MmaBF16 or MmaF16
    typedef typename EL::frag frag;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kAttnBC * kKStride];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][kAttnD * kVtStride];

    // One workgroup per (query block, head), numbered level by level with the
    // heads fastest: level 0 holds every head's longest causal block. The
    // hardware deals workgroup IDs round-robin to its partitions (8 XCDs,
    // each split again), so with the heads fastest every partition gets the
    // same mix of long and short causal blocks, longest first. (Numbered with
    // the query blocks fastest, a multiple of 32 of them put the same block
    // position in the same partition every time, and causal attention took as
    // long as full attention.)
    const int64_t nqb = (a.T + kAttnBQ - 1) / kAttnBQ;
    const int64_t BH = a.B * a.H;
    const int64_t lev = int64_t(blockIdx.x) / BH;
    const int64_t bh = int64_t(blockIdx.x) - lev * BH;
    const int64_t qblk = a.causal ? nqb - 1 - lev : lev;
    const int64_t b = bh / a.H, h = bh % a.H;
    const uint16_t* Q = a.q + b * a.qb + h * a.qh;
    const uint16_t* Kg = a.k + b * a.kb + h * a.kh;
    const uint16_t* Vg = a.v + b * a.vb + h * a.vh;
    uint16_t* O = a.o + b * a.ob + h * a.oh;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int g = lane / 32;
    const int64_t q0 = qblk * kAttnBQ + wave * 32;
    const int64_t myq = q0 + lane % 32;  // the query of this lane

    // Q^T fragments (B operand): query myq, dims kk * 16 + g * 8 + e
    frag qf[kAttnD / 16];
#pragma unroll
    for (int kk = 0; kk < kAttnD / 16; ++kk) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (myq < a.T) w = *reinterpret_cast<const u32x4*>(Q + myq * a.qt + kk * 16 + g * 8);
        qf[kk] = __builtin_bit_cast(frag, w);
    }

    // key blocks to visit: all, or up to the block's last query when causal
    const int64_t q_last = (qblk + 1) * kAttnBQ < a.T ? (qblk + 1) * kAttnBQ : a.T;
    const int64_t kend = a.causal ? q_last : a.T;
    const int64_t nkb = (kend + kAttnBC - 1) / kAttnBC;

    // Staging. K: thread tid moves chunks c = tid + i * threads (key c / 16,
    // dims (c % 16) * 8 .. + 8), stored row-major. V is stored transposed
    // (V^T[dim][key]); thread tid takes the key pair 2 p, 2 p + 1
    // (p = tid % 32) and dims 8 (tid / 32 + 8 i) .. + 8, and writes each dim
    // of the pair as one 32-bit word: the 64 lanes of a wave then write 32
    // consecutive words of one V^T row and 32 of the row 8 dims further
    // (1152 bytes apart, the other half of the banks), without conflicts.
    constexpr int kVPairs = kAttnBC / 2;                            // 32 key pairs
    constexpr int kVRounds = (kAttnD / 8) / (kAttnThreads / kVPairs);  // dim blocks per thread
    u32x4 rk[kAttnLoads], rv[2 * kVRounds];
    auto load_block = [&](int64_t kb0) {
#pragma unroll
        for (int i = 0; i < kAttnLoads; ++i) {
            const int c = tid + i * kAttnThreads;
            const int64_t key = kb0 + c / (kAttnD / 8);
            const int dim = (c % (kAttnD / 8)) * 8;
            rk[i] = key < a.T ? *reinterpret_cast<const u32x4*>(Kg + key * a.kt + dim)
                              : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < kVRounds; ++i) {
            const int64_t key = kb0 + 2 * (tid % kVPairs);
            const int dim = 8 * (tid / kVPairs + i * (kAttnThreads / kVPairs));
            rv[2 * i] = key < a.T ? *reinterpret_cast<const u32x4*>(Vg + key * a.vt + dim)
                                  : u32x4{0u, 0u, 0u, 0u};
            rv[2 * i + 1] = key + 1 < a.T
                                ? *reinterpret_cast<const u32x4*>(Vg + (key + 1) * a.vt + dim)
                                : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_block = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kAttnLoads; ++i) {
            const int c = tid + i * kAttnThreads;
            const int key = c / (kAttnD / 8);
            const int dim = (c % (kAttnD / 8)) * 8;
            *reinterpret_cast<u32x4*>(&Ks[buf][key * kKStride + dim]) = rk[i];
        }
#pragma unroll
        for (int i = 0; i < kVRounds; ++i) {
            const int key = 2 * (tid % kVPairs);
            const int dim = 8 * (tid / kVPairs + i * (kAttnThreads / kVPairs));
            const uint32_t a0[4] = {rv[2 * i].x, rv[2 * i].y, rv[2 * i].z, rv[2 * i].w};
            const uint32_t a1[4] = {rv[2 * i + 1].x, rv[2 * i + 1].y, rv[2 * i + 1].z,
                                    rv[2 * i + 1].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // dims dim + 2e (low halves) and dim + 2e + 1 (high halves)
                *reinterpret_cast<uint32_t*>(&Vt[buf][(dim + 2 * e) * kVtStride + key]) =
                    (a0[e] & 0xFFFFu) | (a1[e] << 16);
                *reinterpret_cast<uint32_t*>(&Vt[buf][(dim + 2 * e + 1) * kVtStride + key]) =
                    (a0[e] >> 16) | (a1[e] & 0xFFFF0000u);
            }
        }
    };

    f32x16 acc[kAttnD / 32];  // O^T: rows dt * 32 + (v / 4) * 8 + 4 g + v % 4, column myq
#pragma unroll
    for (int dt = 0; dt < kAttnD / 32; ++dt) acc[dt] = f32x16{};
    float m = -__builtin_inff();
    float l = 0.0f;

    load_block(0);
    store_block(0);
    __syncthreads();
    for (int64_t kb = 0; kb < nkb; ++kb) {
        const int buf = static_cast<int>(kb & 1);
        const int64_t kb0 = kb * kAttnBC;
        if (kb + 1 < nkb) load_block(kb0 + kAttnBC);

        // a causal block wholly above this wave's queries contributes nothing
        // (its last key block can be): the wave skips it (uniform branch)
        if (!(a.causal && kb0 > q0 + 31)) {
            // S^T for the block's two 32-key tiles; the tiles alternate so
            // that consecutive MFMAs are independent (a lone tile is a chain
            // of 8 dependent MFMAs, each also waiting on its LDS read)
            f32x16 s[2] = {f32x16{}, f32x16{}};
            const uint16_t* kbase = &Ks[buf][(lane % 32) * kKStride + g * 8];
#pragma unroll
            for (int kk = 0; kk < kAttnD / 16; ++kk)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    s[t] = EL::mfma(
                        *reinterpret_cast<const frag*>(kbase + t * 32 * kKStride + kk * 16),
                        qf[kk], s[t]);

            // mask (only blocks that reach past T or, causal, past the wave's
            // first query), then the block max over the query's 32 keys, in
            // raw score units (the scale is positive)
            if (kb0 + kAttnBC > a.T || (a.causal && kb0 + kAttnBC - 1 > q0)) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int64_t key = kb0 + t * 32 + (v / 4) * 8 + g * 4 + v % 4;
                        if (key >= a.T || (a.causal && key > myq)) s[t][v] = -__builtin_inff();
                    }
                }
            }
            float bm = -__builtin_inff();
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v) bm = fmaxf(bm, s[t][v]);
            bm = fmaxf(bm, __shfl_xor(bm, 32)) * a.scale_log2;
            const float mn = fmaxf(m, bm);
            // while every key seen is masked (mn = -inf) nothing accumulates
            const float base = mn == -__builtin_inff() ? 0.0f : mn;
            const float corr = (m == mn) ? 1.0f : exp2_raw(m - base);
            float bs = 0.0f;
            frag pf[4];  // P^T fragments: chunk 2 t + c of tile t
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float pv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        // 2^(s scale - base): the scale folded into one fma
                        pv[e] = exp2_raw(fmaf(s[t][c * 8 + e], a.scale_log2, -base));
                        bs += pv[e];
                    }
                    u32x4 w;
                    w.x = EL::cvt2(pv[0], pv[1]);
                    w.y = EL::cvt2(pv[2], pv[3]);
                    w.z = EL::cvt2(pv[4], pv[5]);
                    w.w = EL::cvt2(pv[6], pv[7]);
                    pf[t * 2 + c] = __builtin_bit_cast(frag, w);
                }
            }
            bs += __shfl_xor(bs, 32);
            l = l * corr + bs;
            // rescale the accumulators only when some lane's max grew (after
            // the first blocks it rarely does; multiplying by 1 is a no-op)
            if (__builtin_amdgcn_ballot_w64(m != mn) != 0) {
#pragma unroll
                for (int dt = 0; dt < kAttnD / 32; ++dt) acc[dt] *= corr;
            }
            m = mn;

            // O^T += V^T P^T; V^T fragment of d-tile dt, chunk (t, c): dims
            // dt * 32 + lane % 32, keys t * 32 + 16 c + 4 g + {0..3} and + 8,
            // read as two 8-byte runs (pairs of keys per 32-bit word)
            // (key chunks outer, the four independent d-tiles inner)
            const uint16_t* vbase = &Vt[buf][(lane % 32) * kVtStride + 4 * g];
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                const int k0 = (ch / 2) * 32 + (ch % 2) * 16;
#pragma unroll
                for (int dt = 0; dt < kAttnD / 32; ++dt) {
                    const uint16_t* vrow = vbase + dt * 32 * kVtStride;
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + k0);
                    const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + k0 + 8);
                    const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
                    acc[dt] = EL::mfma(__builtin_bit_cast(frag, w), pf[ch], acc[dt]);
                }
            }
        }

        if (kb + 1 < nkb) store_block(buf ^ 1);
        __syncthreads();
    }

    // O = acc / l, rounded to bf16; four consecutive dims per 8-byte store
    if (myq < a.T) {
        const float r = 1.0f / l;
        uint16_t* orow = O + myq * a.ot;
#pragma unroll
        for (int dt = 0; dt < kAttnD / 32; ++dt) {
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int d = dt * 32 + v4 * 8 + g * 4;
                uint32_t w0 = EL::cvt2(acc[dt][v4 * 4 + 0] * r, acc[dt][v4 * 4 + 1] * r);
                uint32_t w1 = EL::cvt2(acc[dt][v4 * 4 + 2] * r, acc[dt][v4 * 4 + 3] * r);
                *reinterpret_cast<uint64_t*>(orow + d) = uint64_t(w0) | (uint64_t(w1) << 32);
            }
        }
    }
}

}  // namespace fk
