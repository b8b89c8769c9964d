// device_common.hpp -- device-side building blocks shared by the kernels of
// libfusedops (gfx950 only): 16-byte vector I/O for fp32 and bf16, the
// tanh-GELU in exp2 form, and wave64 reductions through DPP lane moves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;  // CDNA wavefront width

// ------------------------------------------------------------------ I/O ---
// Each storage type describes how 16 bytes (one global_load_dwordx4 per
// lane) unpack into fp32 values and back.

struct IoF32 {
    static constexpr int kVec = 4;  // elements per 16 bytes
    static constexpr int kBytes = 4;
    __device__ static inline void unpack(const u32x4 w, float* v) {
        v[0] = __uint_as_float(w.x);
        v[1] = __uint_as_float(w.y);
        v[2] = __uint_as_float(w.z);
        v[3] = __uint_as_float(w.w);
    }
    __device__ static inline u32x4 pack(const float* v) {
        u32x4 w;
        w.x = __float_as_uint(v[0]);
        w.y = __float_as_uint(v[1]);
        w.z = __float_as_uint(v[2]);
        w.w = __float_as_uint(v[3]);
        return w;
    }
    __device__ static inline float load1(const void* p, int64_t i) {
        return static_cast<const float*>(p)[i];
    }
    __device__ static inline void store1(void* p, int64_t i, float v) {
        static_cast<float*>(p)[i] = v;
    }
};

struct IoBF16 {
    static constexpr int kVec = 8;
    static constexpr int kBytes = 2;
    // bf16 -> fp32 is exact: the bf16 bits are the upper half of the fp32.
    __device__ static inline float lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ static inline float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
    // fp32 pair -> packed bf16 pair, nearest even (one v_cvt_pk_bf16_f32).
    __device__ static inline uint32_t cvt2(float a, float b) {
        f32x2 f = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
    }
    __device__ static inline void unpack(const u32x4 w, float* v) {
        v[0] = lo(w.x); v[1] = hi(w.x);
        v[2] = lo(w.y); v[3] = hi(w.y);
        v[4] = lo(w.z); v[5] = hi(w.z);
        v[6] = lo(w.w); v[7] = hi(w.w);
    }
    __device__ static inline u32x4 pack(const float* v) {
        u32x4 w;
        w.x = cvt2(v[0], v[1]);
        w.y = cvt2(v[2], v[3]);
        w.z = cvt2(v[4], v[5]);
        w.w = cvt2(v[6], v[7]);
        return w;
    }
    __device__ static inline float load1(const void* p, int64_t i) {
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
    }
    __device__ static inline void store1(void* p, int64_t i, float v) {
        static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(cvt2(v, 0.0f) & 0xFFFFu);
    }
};

// 16-bit element types on the matrix cores (the Linear and attention
// kernels): the MFMA operand vector (8 elements = 16 bytes), the 32x32x16
// MFMA with fp32 accumulation, fp32 pairs -> two packed elements rounded to
// nearest even, and single-element loads and stores.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct MmaBF16 {
    typedef bf16x8 frag;
    __device__ static inline f32x16 mfma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline uint32_t cvt2(float a, float b) { return IoBF16::cvt2(a, b); }
    __device__ static inline float load1(const void* p, int64_t i) { return IoBF16::load1(p, i); }
    __device__ static inline void store1(void* p, int64_t i, float v) { IoBF16::store1(p, i, v); }
};
struct MmaF16 {
    typedef f16x8 frag;
    __device__ static inline f32x16 mfma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static inline uint32_t cvt2(float a, float b) {
        f32x2 f = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
    }
    __device__ static inline float load1(const void* p, int64_t i) {
        return static_cast<float>(static_cast<const _Float16*>(p)[i]);
    }
    __device__ static inline void store1(void* p, int64_t i, float v) {
        static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(cvt2(v, 0.0f) & 0xFFFFu);
    }
};

// 16-byte global load/store; NT selects the non-temporal (streaming) hint.
template <bool NT>
__device__ inline u32x4 ld16(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ inline void st16(u32x4* p, u32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// ---------------------------------------------------------------- math ---
constexpr float kLog2e = 1.4426950408889634f;

// Raw hardware 2^a (v_exp_f32). Results below 2^-126 come back as zero, which
// is harmless where they only feed a sum that is at least 1.
__device__ inline float exp2_raw(float a) { return __builtin_amdgcn_exp2f(a); }

// Softmax numerators are computed as e' = 2^(a + kSoftmaxBias), a = (x - m)
// log2(e) <= 0, and normalised by the sum of the same e'; the common factor
// 2^kSoftmaxBias cancels exactly (a power of two). The bias keeps e' normal
// down to a = -134: any smaller numerator gives an output below 2^-134,
// which is zero in bf16 (half its smallest subnormal, a tie to even) and
// below 5e-41 in fp32. The bias costs at most 2^-22 of rounding on the
// exponent argument (its magnitude stays below 8 for the numerators that
// matter), i.e. <= 1.7e-7 relative on e'.
constexpr float kSoftmaxBias = 8.0f;
constexpr float kSoftmaxScale = 256.0f;  // 2^kSoftmaxBias

// e' for one element: one subtraction, one fused multiply-add, one exp.
__device__ inline float softmax_numerator(float x, float m) {
    return exp2_raw(fmaf(x - m, kLog2e, kSoftmaxBias));
}

// tanh-GELU: 0.5 x (1 + tanh u), u = sqrt(2/pi) (x + 0.044715 x^3)
// (the GELU case of the "CS336 lecture 6" notes, section 4.2).
// With 1 + tanh u = 2 / (1 + e^(-2u)) this is x / (1 + 2^t) where
// t = -2u log2(e) = x (A + B x^2), A = -2 sqrt(2/pi) log2(e) and
// B = 0.044715 A: one exp2 and one reciprocal, and no cancellation for
// negative x (the literal form loses all digits below x ~ -3 in fp32).
constexpr float kGeluA = -2.302208198144325f;    // -2 * sqrt(2/pi) * log2(e)
constexpr float kGeluB = -0.10294323958002348f;  // 0.044715 * kGeluA
// Above this t (x below ~ -9.5) 1 + 2^t is 2^t to fp32 precision and its
// reciprocal would leave the normal range; those lanes take the far path.
constexpr float kGeluFarT = 120.0f;

__device__ inline float gelu_t(float x) { return x * fmaf(kGeluB, x * x, kGeluA); }

// x * 2^-t, scaled so that no intermediate is subnormal; the limit -0 at -inf.
__device__ inline float gelu_far(float x, float t) {
    const float y = (x * exp2_raw(64.0f - t)) * 0x1p-64f;
    return x == -__builtin_inff() ? -0.0f : y;
}

// GELU over N values in registers. The common path is branch-free; lanes
// with t > kGeluFarT are patched under one wave-uniform branch (a ballot),
// so the fast path never diverges. NaN stays NaN, +inf -> +inf,
// -inf -> -0, +-0 -> +-0.
template <int N>
__device__ inline void gelu_tanh_n(float (&v)[N]) {
    float t[N];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < N; ++j) {
        t[j] = gelu_t(v[j]);
        tmax = fmaxf(tmax, t[j]);
    }
    float y[N];
#pragma unroll
    for (int j = 0; j < N; ++j) y[j] = v[j] * __builtin_amdgcn_rcpf(1.0f + exp2_raw(t[j]));
    if (__builtin_amdgcn_ballot_w64(tmax > kGeluFarT) != 0) {
        // every value's far form, then a select: one compare mask live at a
        // time (a branch per value kept all N masks in SGPR pairs at once)
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const float yf = gelu_far(v[j], t[j]);
            y[j] = t[j] > kGeluFarT ? yf : y[j];
        }
    }
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = y[j];
}

// ReLU: v for v > 0, else +0; NaN stays NaN (as torch's relu).
__device__ inline float relu1(float v) { return (v > 0.0f || v != v) ? v : 0.0f; }

// Derivative of the tanh-GELU (for the backward pass; derived from the
// forward definition): with s = 1 / (1 + 2^t) (the logistic of 2u) and
// q = 1 - s, GELU'(x) = s + w s q, w = 2 sqrt(2/pi) x (1 + 3 * 0.044715 x^2).
// q is formed without cancellation: 1 - s where s < 1/2 (t > 0), e s where
// e = 2^t <= 1. Where s q is 0 (large |x|) the second term is dropped
// (avoids 0 * inf), giving the limits 1 at +inf and 0 at -inf.
constexpr float kGeluW0 = 1.5957691216057308f;    // 2 sqrt(2/pi)
constexpr float kGeluW1 = 0.21406444881780076f;   // 6 sqrt(2/pi) 0.044715

// g[j] <- g[j] * GELU'(x[j]) for N values in registers; far-negative lanes
// (t > kGeluFarT) are patched under one wave-uniform branch as in
// gelu_tanh_n, with s = 2^-t formed as 2^(64 - t) 2^-64.
template <int N>
__device__ inline void gelu_tanh_grad_n(const float (&x)[N], float (&g)[N]) {
    float t[N];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < N; ++j) {
        t[j] = gelu_t(x[j]);
        tmax = fmaxf(tmax, t[j]);
    }
    float r[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const float e = exp2_raw(t[j]);
        const float s = __builtin_amdgcn_rcpf(1.0f + e);
        const float q = t[j] > 0.0f ? 1.0f - s : e * s;
        const float w = x[j] * fmaf(kGeluW1, x[j] * x[j], kGeluW0);
        const float sq = s * q;
        const float d = sq == 0.0f ? s : fmaf(w, sq, s);
        r[j] = g[j] * d;
    }
    if (__builtin_amdgcn_ballot_w64(tmax > kGeluFarT) != 0) {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            if (t[j] > kGeluFarT) {
                const float s = exp2_raw(64.0f - t[j]);  // 2^64 GELU'-scale factor
                const float w = x[j] * fmaf(kGeluW1, x[j] * x[j], kGeluW0);
                const float d = s == 0.0f ? 0.0f : s * (1.0f + w);
                r[j] = (g[j] * d) * 0x1p-64f;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < N; ++j) g[j] = r[j];
}

// ------------------------------------------------------- wave reductions --
// DPP lane moves within a wave64: quad_perm swaps within 4 lanes,
// row_half_mirror reverses 8 lanes, row_mirror reverses 16 lanes. After the
// four steps every lane of a 16-lane row holds that row's result; the four
// row results are then read as scalars and combined in a fixed order, so
// the reduction is deterministic and every lane gets the same bits.
enum : int {
    kDppQuadSwap1 = 0xB1,  // quad_perm [1,0,3,2]
    kDppQuadSwap2 = 0x4E,  // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141,
    kDppMirror = 0x140,
};

template <int kCtrl>
__device__ inline float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

__device__ inline float lane_value(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// All 64 lanes must be active.
__device__ inline float wave_max(float v) {
    v = fmaxf(v, dpp<kDppQuadSwap1>(v));
    v = fmaxf(v, dpp<kDppQuadSwap2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    v = fmaxf(v, dpp<kDppMirror>(v));
    return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)),
                 fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

__device__ inline float wave_sum(float v) {
    v = v + dpp<kDppQuadSwap1>(v);
    v = v + dpp<kDppQuadSwap2>(v);
    v = v + dpp<kDppHalfMirror>(v);
    v = v + dpp<kDppMirror>(v);
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Online-softmax state merge (running max m, running sum l of 2^((x - m) L),
// L = log2 e): the larger max wins and the other sum is rescaled by
// 2^((m_i - m) L). Symmetric in its operands, so both partners of a lane
// exchange agree; equal maxima (including two empty states, m = -inf) keep
// factor 1.
__device__ inline void ml_merge(float& m, float& l, float m2, float l2) {
    const float mn = fmaxf(m, m2);
    const float f1 = (m == mn) ? 1.0f : exp2_raw((m - mn) * kLog2e);
    const float f2 = (m2 == mn) ? 1.0f : exp2_raw((m2 - mn) * kLog2e);
    l = l * f1 + l2 * f2;
    m = mn;
}

template <int kCtrl>
__device__ inline void ml_dpp_step(float& m, float& l) {
    ml_merge(m, l, dpp<kCtrl>(m), dpp<kCtrl>(l));
}

// All 64 lanes must be active; returns the wave's merged (m, l) in every lane.
__device__ inline void wave_ml(float& m, float& l) {
    ml_dpp_step<kDppQuadSwap1>(m, l);
    ml_dpp_step<kDppQuadSwap2>(m, l);
    ml_dpp_step<kDppHalfMirror>(m, l);
    ml_dpp_step<kDppMirror>(m, l);
    float m0 = lane_value(m, 0), l0 = lane_value(l, 0);
    float m1 = lane_value(m, 16), l1 = lane_value(l, 16);
    float m2 = lane_value(m, 32), l2 = lane_value(l, 32);
    float m3 = lane_value(m, 48), l3 = lane_value(l, 48);
    ml_merge(m0, l0, m1, l1);
    ml_merge(m2, l2, m3, l3);
    ml_merge(m0, l0, m2, l2);
    m = m0;
    l = l0;
}

}  // namespace fk
