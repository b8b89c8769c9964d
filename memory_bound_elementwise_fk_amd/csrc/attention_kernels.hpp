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
// MI355X mapping. Each wave owns 32 queries; a workgroup of 8 waves (or 4,
// for grids too small to fill the GPU) owns 256 (128) queries of one
// (batch, head) and walks the key blocks of 64 keys,
// staged through LDS (K and V both as [key][dim], copied by direct
// global-to-LDS loads: no registers, no ALU; K in three buffers, each
// block loaded two iterations before its scores are computed, V in two, one
// iteration before its P V product, for the software pipeline described at
// the loop). The wave
// computes the transposed scores S^T = K Q^T with the 32x32x16 bf16 MFMA:
// K is the A operand (lane l: key l % 32, dims (l / 32) * 8 + e), Q the B
// operand (query l % 32), staged through LDS once and then held in
// registers for the whole key loop. In the
// accumulator layout of S^T every lane holds one query (l % 32) and 16 of
// the 32 keys of a tile (lane l ^ 32 holds the other 16), so the row max and
// sum of a query are a lane-local reduction plus one exchange with lane
// l ^ 32, and the rescaling of the output accumulator is per lane. The P V
// product is computed as O^T = V^T P^T: P^T is the B operand and comes
// straight from the lane's S^T registers (rounded to bf16) -- the MFMA's
// k index g * 8 + e (g = l / 32) is taken to mean key 8 (e / 4) + 4 g + e % 4
// of each 16-key chunk, which is the order the accumulator layout holds
// them in. V^T's A fragments (lane l: dim l % 32, those 8 keys) come from
// the row-major V block through the transposing LDS read of gfx950
// (ds_read_b64_tr_b16): in each group of 16 lanes, lane 4a + b receives
// element b of the 8-byte runs that lanes a, a + 4, a + 8, a + 12 address
// (checked on the device), so lanes pointing at 4 consecutive keys of one
// 4-dim run hand every lane 4 consecutive keys of its dim -- two such reads
// per fragment. The output accumulator O^T again holds one query per lane,
// so the final division by l is per lane.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "gemm_kernels.hpp"

namespace fk {

constexpr int kAttnD = 128;       // head dimension
constexpr int kAttnBC = 64;       // keys per block
constexpr int kAttnWaveQ = 32;    // queries per wave
constexpr int kAttnRowBytes = kAttnD * 2;                       // one key row of K or V
constexpr int kAttnBlockBytes = kAttnBC * kAttnRowBytes;        // 16 KiB per operand
// queries per workgroup of NW waves (4 or 8)
template <int NW>
constexpr int kAttnBQ = NW * kAttnWaveQ;
// the 4-wave shape has the most workgroups: the grid-size limit uses it
constexpr int kAttnBQMin = kAttnBQ<4>;
// LDS layout of a block: row r (key) holds its 16 chunks of 16 bytes (8
// dims each) permuted, chunk c at position c ^ swz(r): K with r % 16 (the
// S^T fragment reads, 16 consecutive keys of one chunk per 256 bytes, hit
// all 64 banks), V with 4 (r % 4) (the transposing reads, 4 consecutive
// keys x 4 chunks per 256 bytes, hit all 64 banks).
__device__ inline int attn_swz_k(int r) { return r & 15; }
__device__ inline int attn_swz_v(int r) { return (r & 3) * 4; }
// The running max m moves only when a block's max exceeds it by more than
// this (log2 units): the numerators 2^(s - m) then stay below 2^8, and the
// output acc / l does not depend on which m was subtracted, so it is the
// same softmax. Random scores raise the max in most blocks by a little; each
// raise costs a rescale of the 64 accumulator values of the lane.
constexpr float kAttnMaxSlack = 8.0f;

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
    // heads per group of the workgroup order (0: one group of all heads);
    // > 0 only when B H is a multiple of 8 and (B H / 8) % hgroup == 0
    int64_t hgroup;
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// transposing 8-byte LDS read (see the lane rule above)
__device__ inline u32x2 lds_read_tr16(const uint16_t* p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// Two waves per SIMD: with one, a wave's MFMA, exponential and LDS phases
// run back to back and the K/V loads barely overlap them; the second wave
// fills those gaps. The kernel fits in the 256 registers (no AGPRs) this
// leaves a wave. NW = 8: one workgroup per CU, whose 8 waves share each
// K/V block (half the direct-load traffic per query of NW = 4, where two
// workgroups of 4 waves share a CU, LDS 80 KiB each).
template <class EL, bool WIDE, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attention_fwd_kernel(AttnArgs a) {  // EL: MmaBF16 or MmaF16
    typedef typename EL::frag frag;
    static_assert(NW == 4 || NW == 8, "workgroups of 4 or 8 waves");
    constexpr int kBQ = kAttnBQ<NW>;
    // direct loads per wave, per operand and block (each fills 1 KiB = 4 rows)
    constexpr int kDmaPerWave = kAttnBlockBytes / 1024 / NW;
    static_assert(kDmaPerWave * 1024 * NW == kAttnBlockBytes, "whole wave loads");
    // K in three buffers (kv[0..2]), V in two (kv[3..4]): 80 KiB, two 4-wave
    // workgroups fill a CU's LDS; after the key loop, the output's staging
    constexpr int kKBuf0 = 0, kVBuf0 = 3;
    __shared__ __attribute__((aligned(1024))) uint16_t kv[5][kAttnBC * kAttnD];

    // One workgroup per (query block, head). The hardware deals workgroup
    // IDs round-robin to its partitions: ID mod 8 picks the XCD (each with
    // its own L2), and each XCD splits its share again. The IDs go level by
    // level, a level holding one query block of every head in a group, with
    // the heads fastest: for causal attention level 0 holds the longest
    // blocks, so every partition gets the same mix of long and short blocks,
    // longest first. (Numbered with the query blocks fastest, a multiple of
    // 32 of them put the same block position in the same partition every
    // time, and causal attention took as long as full attention.) When B H
    // is a multiple of 8 (hgroup > 0), XCD x takes heads x, x + 8, ... in
    // groups of hgroup heads: the workgroups running together on an XCD then
    // share few heads and read each K and V block from its L2 rather than
    // from HBM. Full attention takes one head per group, so all of a head's
    // query blocks run together; causal attention groups up to 4 heads,
    // which keeps most of the longest-first order. Otherwise all heads form
    // one group.
    //
    // Positions, counts and this mapping are 32-bit: the launcher keeps the
    // grid at most 2^23 workgroups of at least 128 queries, so T <= 2^30
    // and B H, the query blocks and the IDs stay below 2^23. (In 64 bits
    // the divisions below took ~500 scalar instructions per wave, which the
    // waves of a CU issue through one shared scalar unit: ~3 us per
    // workgroup before its first load.) Element offsets stay 64-bit.
    const int32_t T = static_cast<int32_t>(a.T);
    const uint32_t nqb = (static_cast<uint32_t>(T) + kBQ - 1) / kBQ;
    const uint32_t BH = static_cast<uint32_t>(a.B * a.H);
    const uint32_t bid = blockIdx.x;
    uint32_t bh, qblk;
    if (a.hgroup > 0) {
        const uint32_t hg = static_cast<uint32_t>(a.hgroup);
        const uint32_t x = bid % 8, k = bid / 8;  // the XCD's k-th
        const uint32_t per = hg * nqb;
        const uint32_t grp = k / per, r = k - grp * per;
        const uint32_t lev = r / hg;
        bh = (grp * hg + (r - lev * hg)) * 8 + x;
        qblk = a.causal ? nqb - 1 - lev : lev;
    } else {
        const uint32_t lev = bid / BH;
        bh = bid - lev * BH;
        qblk = a.causal ? nqb - 1 - lev : lev;
    }
    const uint32_t H = static_cast<uint32_t>(a.H);
    const uint32_t b = bh / H, h = bh - b * H;
    const uint16_t* Q = a.q + int64_t(b) * a.qb + int64_t(h) * a.qh;
    const uint16_t* Kg = a.k + int64_t(b) * a.kb + int64_t(h) * a.kh;
    const uint16_t* Vg = a.v + int64_t(b) * a.vb + int64_t(h) * a.vh;
    uint16_t* O = a.o + int64_t(b) * a.ob + int64_t(h) * a.oh;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int g = lane / 32;
    const int32_t q0 = static_cast<int32_t>(qblk) * kBQ + wave * kAttnWaveQ;
    const int32_t myq = q0 + lane % 32;  // the query of this lane

    // Q^T fragments (B operand): query myq, dims kk * 16 + g * 8 + e; read
    // from the wave's staged Q rows before the key loop
    frag qf[kAttnD / 16];

    // key blocks to visit: all, or up to the block's last query when causal
    const int32_t q_end = (static_cast<int32_t>(qblk) + 1) * kBQ;
    const int32_t q_last = q_end < T ? q_end : T;
    const int32_t kend = a.causal ? q_last : T;
    const int32_t nkb = (kend + kAttnBC - 1) / kAttnBC;

    // Staging: wave w's direct load j (of n per operand: 4 for NW = 4, 2
    // for NW = 8) of a block fills rows 4 u .. 4 u + 3 of K (and of V),
    // u = n w + j; lane i writes position i % 16 of row i / 16 of those, so
    // it fetches the logical chunk at that position. Row r = 4 u + drow has
    // r % 16 = 4 (u % 4) + drow and r % 4 = drow, so the lane's source
    // offset within a block is, for K, r kt + ((dpos ^ drow) 8 ^ 32 (u % 4))
    // and, for V, r vt + (dpos ^ 4 drow) 8. These offsets are lane values
    // kept in vector registers for the whole loop (held as scalars, with
    // the block bases and strides, they pushed the loop past the scalar
    // registers). A block wholly inside T adds them to its first row; the
    // last partial one clamps rows past T to row T - 1 (valid memory; those
    // keys are masked, p = 0). LDS addresses are wave-uniform (scalar).
    const int drow = lane / 16, dpos = lane % 16;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t ks_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((las_ptr)(&kv[kKBuf0][0])));
    const uint32_t vs_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((las_ptr)(&kv[kVBuf0][0])));
    // element offsets within a block: 32-bit unless 64 rows of a stride
    // exceed 2^31 elements (WIDE, chosen on the host)
    typedef typename std::conditional<WIDE, int64_t, int32_t>::type off_t;
    off_t koff[kDmaPerWave], voff[kDmaPerWave];
    int64_t kt_v = a.kt, vt_v = a.vt;  // the strides as lane values (clamped rows)
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
        const int u = wave * kDmaPerWave + j, r = 4 * u + drow;
        koff[j] = static_cast<off_t>(r * a.kt + (((dpos ^ drow) * 8) ^ (32 * (u & 3))));
        voff[j] = static_cast<off_t>(r * a.vt + (dpos ^ attn_swz_v(drow)) * 8);
        asm volatile("" : "+v"(koff[j]), "+v"(voff[j]));
    }
    asm volatile("" : "+v"(kt_v), "+v"(vt_v));
    // the block at key kb0 of K (IS_V false) or V into buffer buf
    auto issue = [&](bool is_v, int32_t kb0, int buf) {
        const bool whole = kb0 + kAttnBC <= T;
        const uint16_t* blk = (is_v ? Vg : Kg) + int64_t(kb0) * (is_v ? a.vt : a.kt);
        const uint32_t lds = (is_v ? vs_base : ks_base) + static_cast<uint32_t>(buf * kAttnBlockBytes);
#pragma unroll
        for (int j = 0; j < kDmaPerWave; ++j) {
            const int u = wave_s * kDmaPerWave + j;
            const uint32_t off = static_cast<uint32_t>(u * 1024);
            const uint16_t* src = blk + (is_v ? voff[j] : koff[j]);
            if (!whole) {
                const int r = (wave * kDmaPerWave + j) * 4 + drow;
                const int32_t rr = kb0 + r < T ? r : T - 1 - kb0;  // row of the block
                src = blk + rr * (is_v ? vt_v : kt_v) +
                      (dpos ^ (is_v ? attn_swz_v(r) : attn_swz_k(r))) * 8;
            }
            lds_dma16(src, lds + off);
        }
    };

    f32x16 acc[kAttnD / 32];  // O^T: rows dt * 32 + (v / 4) * 8 + 4 g + v % 4, column myq
#pragma unroll
    for (int dt = 0; dt < kAttnD / 32; ++dt) acc[dt] = f32x16{};
    float m = -__builtin_inff();
    float l = 0.0f;

    // fragment addressing of this lane: S^T reads key row (t * 32 + lane % 32)
    // at chunk 2 kk + g; the V^T reads (two per fragment) take row k0 + e of
    // 4-dim run 4 a of the lane's 16-dim half, e = (lane % 16) / 4,
    // a = lane % 4, half = (lane / 16) % 2
    const int vt_e = (lane % 16) / 4, vt_a = lane % 4, vt_half = (lane / 16) % 2;

    // S^T of one 64-key block from K buffer kbuf: the block's two 32-key
    // tiles alternate so that consecutive MFMAs are independent (a lone tile
    // is a chain of 8 dependent MFMAs, each also waiting on its LDS read)
    const int kr = lane % 32;  // + t * 32: the same swizzle (r % 16)
    auto compute_s = [&](int kbuf, f32x16 (&s)[2]) {
        s[0] = f32x16{};
        s[1] = f32x16{};
        const uint16_t* kbase = &kv[kKBuf0 + kbuf][kr * kAttnD];
#pragma unroll
        for (int kk = 0; kk < kAttnD / 16; ++kk)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                s[t] = EL::mfma(*reinterpret_cast<const frag*>(
                                    kbase + t * 32 * kAttnD + (((2 * kk + g) ^ attn_swz_k(kr)) * 8)),
                                qf[kk], s[t]);
    };
    // Q staging. Read straight into fragments, each 16-byte load of a wave
    // took 32 bytes from each of 32 rows (32 cache lines for 1 KiB): issuing
    // a workgroup's Q loads took ~2 us. Instead each wave copies its 32 rows
    // (8 KiB) with 8 direct loads of 4 whole rows, laid out like K's rows
    // (chunk c of row r at c ^ (r % 16)), and reads its fragments from LDS.
    // NW = 8: a region of its own (144 KiB of LDS in all, one workgroup per
    // CU). NW = 4 (two workgroups share a CU): K buffer 2 (waves 0, 1) and
    // V buffer 1 (waves 2, 3), which the prologue does not load; K(2) is
    // loaded once every wave has read its Q. Rows past T load row T - 1
    // (valid memory; those queries are not stored).
    uint16_t* qstage;
    if constexpr (NW == 8) {
        __shared__ __attribute__((aligned(1024))) uint16_t qs[NW][kAttnWaveQ * kAttnD];
        qstage = &qs[wave][0];
    } else {
        qstage = wave < 2 ? &kv[kKBuf0 + 2][wave * kAttnWaveQ * kAttnD]
                          : &kv[kVBuf0 + 1][(wave - 2) * kAttnWaveQ * kAttnD];
    }
    auto issue_q = [&]() {
        const uint32_t lds = __builtin_amdgcn_readfirstlane(
            static_cast<uint32_t>(reinterpret_cast<uintptr_t>((las_ptr)(qstage))));
#pragma unroll
        for (int j = 0; j < kAttnWaveQ / 4; ++j) {
            const int r = 4 * j + drow;  // row of the wave's 32; position dpos
            const int32_t row = q0 + r < T ? q0 + r : T - 1;
            lds_dma16(Q + int64_t(row) * a.qt + (dpos ^ attn_swz_k(r)) * 8,
                      lds + static_cast<uint32_t>(j * 1024));
        }
    };
    auto read_q = [&]() {
        const int qr = lane % 32;
#pragma unroll
        for (int kk = 0; kk < kAttnD / 16; ++kk)
            qf[kk] = *reinterpret_cast<const frag*>(qstage + qr * kAttnD +
                                                    (((2 * kk + g) ^ attn_swz_k(qr)) * 8));
    };

    // a causal block wholly above this wave's queries contributes nothing
    // (its last key block can be): the wave skips it (uniform branch)
    auto wave_needs = [&](int32_t kbx) { return !(a.causal && kbx * kAttnBC > q0 + 31); };

    // The mask of block kbx's scores s: only blocks that reach past T or,
    // causal, past the wave's first query have one (a uniform branch).
    auto mask_block = [&](int32_t kbx, f32x16 (&s)[2]) {
        const int32_t kb0 = kbx * kAttnBC;
        if (kb0 + kAttnBC > T || (a.causal && kb0 + kAttnBC - 1 > q0)) {
            // key kb0 + 4 g + off of element (t, v), off = 32 t +
            // 8 (v / 4) + v % 4, is kept while it is at most the last
            // key this query sees (T - 1, or the query when causal)
            const int32_t last = a.causal && myq < T - 1 ? myq : T - 1;
            const int32_t lim = last - kb0 - 4 * g;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (t * 32 + (v / 4) * 8 + v % 4 > lim) s[t][v] = -__builtin_inff();
            }
        }
    };
    // The softmax of a block on its masked scores s, without branches: the
    // block max over the query's 32 keys (raw score units: the scale is
    // positive), the online update of (m, l), and P^T rounded to MFMA
    // fragments. corr and resc tell the P V step of the block how, and
    // whether, to rescale the accumulators first. A block wholly past the
    // wave's keys (T or, causal, its queries) is all masked and changes
    // nothing: bm = -inf keeps m, corr = 1, P = 0.
    auto softmax_block = [&](f32x16 (&s)[2], frag (&pf)[4], float& corr, bool& resc) {
        float bm = -__builtin_inff();
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) bm = fmaxf(bm, s[t][v]);
        bm = fmaxf(bm, __shfl_xor(bm, 32)) * a.scale_log2;
        // the running max moves only for a raise of more than the slack
        // (from -inf, any finite or infinite block max is one)
        const float mn = bm > m + kAttnMaxSlack ? bm : m;
        // while every key seen is masked (mn = -inf) nothing accumulates
        const float base = mn == -__builtin_inff() ? 0.0f : mn;
        corr = (m == mn) ? 1.0f : exp2_raw(m - base);
        float bs = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {  // P^T fragments: chunk 2 t + c of tile t
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
        // the accumulators need a rescale only when some lane's max moved
        // (multiplying by 1 is a no-op)
        resc = __builtin_amdgcn_ballot_w64(m != mn) != 0;
        m = mn;
    };
    // O^T += V^T P^T of block kbx; V^T fragment of d-tile dt, chunk ch:
    // dims dt * 32 + lane % 32, keys 16 ch + 4 g + {0..3} and + 8 (two
    // transposing reads; key chunks outer, the four independent d-tiles
    // inner). Rows k0 + e have e = (k0 + e) % 4, so their swizzle is 4 e.
    auto pv_block = [&](int32_t kbx, const frag (&pf)[4]) {
        const uint16_t* vbuf = &kv[kVBuf0 + (kbx & 1)][0];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            const int k0 = ch * 16 + 4 * g;
#pragma unroll
            for (int dt = 0; dt < kAttnD / 32; ++dt) {
                const int c = dt * 4 + vt_half * 2 + vt_a / 2;  // 16-byte chunk of the run
                const int inner = (vt_a % 2) * 4;              // its 8-byte half
                const int pos = (c ^ (4 * vt_e)) * 8 + inner;
                const u32x2 lo = lds_read_tr16(vbuf + (k0 + vt_e) * kAttnD + pos);
                const u32x2 hi = lds_read_tr16(vbuf + (k0 + 8 + vt_e) * kAttnD + pos);
                const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
                acc[dt] = EL::mfma(__builtin_bit_cast(frag, w), pf[ch], acc[dt]);
            }
        }
    };

    // Software pipeline, two blocks deep: iteration kb masks block kb + 1
    // and rescales the accumulators for block kb (uniform branches), then in
    // one basic block (so that the compiler interleaves the three) adds
    // P(kb) V(kb) (MFMA), runs the softmax of block kb + 1 (VALU) and
    // computes S(kb + 2) (MFMA). With the
    // softmax of a block next to its own P V product (which waits for it),
    // a wave alternated a VALU phase and an MFMA phase, and the per-block
    // barrier kept both waves of a SIMD in the same phase.
    // K block j lives in K buffer j % 3 and V block j in V buffer j % 2.
    // Iteration kb loads V(kb + 1) into the V buffer V(kb - 1) left, then
    // K(kb + 4) into the K buffer K(kb + 1) left (read for S(kb + 1) an
    // iteration earlier). Its closing wait leaves only that K load in
    // flight: the next iteration reads V(kb + 1) and K(kb + 3), loaded an
    // iteration earlier, so K has two iterations to land, V one. One
    // barrier per iteration.
    // Prologue: Q and K(0) first; S(0) waits only for those (the loads
    // land in issue order), while V(0), K(1) and K(2) keep arriving.
    issue_q();
    issue(false, 0, 0);
    issue(true, 0, 0);
    if (nkb > 1) issue(false, kAttnBC, 1);
    if (NW == 8 && nkb > 2) issue(false, 2 * kAttnBC, 2);
    if (NW == 8 && nkb > 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * kDmaPerWave));
    else if (nkb > 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kDmaPerWave));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerWave));
    __syncthreads();
    read_q();
    f32x16 s_cur[2] = {f32x16{}, f32x16{}};
    compute_s(0, s_cur);
    // everything loaded so far has landed, in every wave after the
    // barrier, and every wave has read K(0) (and, NW = 4, its Q, whose
    // buffers K(2) and V(1) take next)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    if (NW == 4 && nkb > 2) issue(false, 2 * kAttnBC, 2);
    if (nkb > 3) issue(false, 3 * kAttnBC, 0);
    frag pf_cur[4];
    float corr_cur;
    bool resc_cur;
    mask_block(0, s_cur);
    softmax_block(s_cur, pf_cur, corr_cur, resc_cur);
    // S(1) (from a stale buffer when there is no block 1: valid LDS, and
    // the block is all masked)
    f32x16 s_nxt[2];
    compute_s(1, s_nxt);
    // K(2) landed (NW = 4; K(3) may still be in flight) and every wave has
    // read K(1) before K(4) replaces it
    if (nkb > 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerWave));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    int kbuf1 = 1, kbuf2 = 2;  // (kb + 1) % 3, (kb + 2) % 3
    for (int32_t kb = 0; kb < nkb; ++kb) {
        if (kb + 1 < nkb) issue(true, (kb + 1) * kAttnBC, (kb + 1) & 1);
        const bool load_k = kb + 4 < nkb;
        if (load_k) issue(false, (kb + 4) * kAttnBC, kbuf1);
        // a causal wave computes nothing past its queries' last block (the
        // later blocks lie past them too); its step at that block runs the
        // softmax of the next block, all masked, and a discarded S
        if (wave_needs(kb)) {
            mask_block(kb + 1, s_nxt);
            if (resc_cur) {
#pragma unroll
                for (int dt = 0; dt < kAttnD / 32; ++dt) acc[dt] *= corr_cur;
            }
            pv_block(kb, pf_cur);
            frag pf_nxt[4];
            float corr_nxt;
            bool resc_nxt;
            softmax_block(s_nxt, pf_nxt, corr_nxt, resc_nxt);
            // S(kb + 2); past the last block it reads a stale buffer (valid
            // LDS) and is discarded
            f32x16 s_new[2];
            compute_s(kbuf2, s_new);
#pragma unroll
            for (int i = 0; i < 4; ++i) pf_cur[i] = pf_nxt[i];
            corr_cur = corr_nxt;
            resc_cur = resc_nxt;
            s_nxt[0] = s_new[0];
            s_nxt[1] = s_new[1];
        }
        // the loads the next iteration reads have landed (this iteration's
        // K loads may still be in flight); after the barrier every wave's
        // have, and the buffers read in this iteration are free
        if (load_k) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerWave));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        kbuf1 = kbuf2;
        kbuf2 = kbuf2 == 2 ? 0 : kbuf2 + 1;
    }

    // O = acc / l, rounded to bf16. A lane holds one query's row (four
    // consecutive dims per (dt, v4)), so stores straight from the registers
    // would touch 32 rows per instruction; the wave stages its 32 rows in
    // LDS (rows padded to 272 bytes: the 8-byte writes of 32 rows spread
    // over the banks) and stores whole 256-byte rows, 16 lanes per row,
    // 16 bytes per lane. The key loop's closing barrier has freed the K/V
    // buffers (8 waves x 8.5 KiB fit in their 80 KiB).
    {
        constexpr int kRow = kAttnD + 8;  // staged row, elements
        static_assert(NW * kAttnWaveQ * kRow * 2 <= int(sizeof(kv)), "output staging fits");
        // (the lane index made opaque here: the addresses below are then
        // computed after the loop rather than kept in registers across it)
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        uint16_t* stage = &kv[0][0] + wave * (kAttnWaveQ * kRow);
        const float r = 1.0f / l;
        const int q = lane_e % 32;
#pragma unroll
        for (int dt = 0; dt < kAttnD / 32; ++dt) {
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int d = dt * 32 + v4 * 8 + g * 4;
                const uint32_t w0 = EL::cvt2(acc[dt][v4 * 4 + 0] * r, acc[dt][v4 * 4 + 1] * r);
                const uint32_t w1 = EL::cvt2(acc[dt][v4 * 4 + 2] * r, acc[dt][v4 * 4 + 3] * r);
                *reinterpret_cast<uint64_t*>(stage + q * kRow + d) = uint64_t(w0) | (uint64_t(w1) << 32);
            }
        }
        // the wave reads rows other lanes wrote
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < kAttnWaveQ / 4; ++i) {
            const int row = i * 4 + lane_e / 16, c = lane_e % 16;
            const u32x4 val = *reinterpret_cast<const u32x4*>(stage + row * kRow + c * 8);
            if (q0 + row < T) *reinterpret_cast<u32x4*>(O + int64_t(q0 + row) * a.ot + c * 8) = val;
        }
    }
}

}  // namespace fk
