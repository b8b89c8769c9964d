// elementwise.hip -- launchers of the streaming kernels in ew_kernels.hpp:
// tanh-GELU, the fused op chain and the byte copy.
#include "ew_kernels.hpp"

namespace fk {
namespace {

// grid * block stays below 2^31 work-items; larger inputs grid-stride.
constexpr int64_t kMaxWorkItems = int64_t(1) << 31;

template <class... Args>
hipError_t launch_kernel(const void* fn, int64_t grid, int block, hipStream_t s, Args... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(block), argv, 0, s);
}

int64_t grid_for(int64_t tiles, int threads) {
    const int64_t cap = kMaxWorkItems / threads;
    return tiles < 1 ? 1 : (tiles > cap ? cap : tiles);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launch shapes (workgroup size T, 16-byte vectors per lane U, non-temporal
// loads/stores), chosen by measurement on MI355X over 2 GiB streams (three
// rounds, every T in {64, 128, 256} x U in {1, 2, 4} x store hint): one
// vector per lane in small workgroups wins -- bf16 GELU 128 x 1 at
// 6.71 TB/s, fp32 GELU 64 x 1 at 6.70 TB/s, copy 64 x 1 at 6.67 TB/s --
// and non-temporal hints help since nothing is re-read. The 32 MiB chain
// (C3) is also fastest at 64 x 1.
template <class IO>
struct EwShape {
    static constexpr int T = IO::kBytes == 2 ? 128 : 64;
    static constexpr int U = 1;
    static constexpr bool NT = true;
};
constexpr int kCopyT = 64, kCopyU = 1;
constexpr bool kCopyNT = true;
constexpr int kScalarT = 256, kScalarPer = 8;

template <class IO, class Op>
hipError_t launch_ew(const void* x, void* y, int64_t n, const Op& op, hipStream_t s) {
    if (aligned16(x) && aligned16(y)) {
        using S = EwShape<IO>;
        const int64_t tile_vec = int64_t(S::T) * S::U;
        const int64_t nfull = (n / IO::kVec) / tile_vec;
        const int64_t ntiles = (n + tile_vec * IO::kVec - 1) / (tile_vec * IO::kVec);
        const auto* xv = static_cast<const u32x4*>(x);
        auto* yv = static_cast<u32x4*>(y);
        if (ntiles <= kMaxWorkItems / S::T)
            return launch_kernel(
                reinterpret_cast<const void*>(&ew_vec_kernel<IO, S::T, S::U, S::NT, false, Op>),
                ntiles, S::T, s, xv, yv, n, nfull, op);
        return launch_kernel(
            reinterpret_cast<const void*>(&ew_vec_kernel<IO, S::T, S::U, S::NT, true, Op>),
            grid_for(ntiles, S::T), S::T, s, xv, yv, n, nfull, op);
    }
    const int64_t tile = int64_t(kScalarT) * kScalarPer;
    return launch_kernel(reinterpret_cast<const void*>(&ew_scalar_kernel<IO, kScalarT, kScalarPer, Op>),
                         grid_for((n + tile - 1) / tile, kScalarT), kScalarT, s, x, y, n, op);
}

template <class IO, int K0, int K1, int K2>
hipError_t launch_aaa(const void* x, void* y, int64_t n, const OpList& ops, hipStream_t s) {
    return launch_ew<IO>(x, y, n, AffActAffOp<K0, K1, K2>{ops.scalar[0], ops.scalar[2]}, s);
}

// The fixed-kind kernel of an "add/mul, GELU/ReLU, add/mul" list.
template <class IO>
hipError_t launch_aaa_family(const void* x, void* y, int64_t n, const OpList& ops, hipStream_t s) {
    const bool add0 = ops.kind[0] == kOpAdd, gelu = ops.kind[1] == kOpGelu,
               add2 = ops.kind[2] == kOpAdd;
    if (add0) {
        if (gelu) return add2 ? launch_aaa<IO, kOpAdd, kOpGelu, kOpAdd>(x, y, n, ops, s)
                              : launch_aaa<IO, kOpAdd, kOpGelu, kOpMul>(x, y, n, ops, s);
        return add2 ? launch_aaa<IO, kOpAdd, kOpRelu, kOpAdd>(x, y, n, ops, s)
                    : launch_aaa<IO, kOpAdd, kOpRelu, kOpMul>(x, y, n, ops, s);
    }
    if (gelu) return add2 ? launch_aaa<IO, kOpMul, kOpGelu, kOpAdd>(x, y, n, ops, s)
                          : launch_aaa<IO, kOpMul, kOpGelu, kOpMul>(x, y, n, ops, s);
    return add2 ? launch_aaa<IO, kOpMul, kOpRelu, kOpAdd>(x, y, n, ops, s)
                : launch_aaa<IO, kOpMul, kOpRelu, kOpMul>(x, y, n, ops, s);
}

bool is_scalar_op(int32_t k) { return k == kOpAdd || k == kOpMul; }
bool is_activation(int32_t k) { return k == kOpGelu || k == kOpRelu; }

// One of the fixed-kind three-op chains.
bool chain_is_aaa(const OpList& ops) {
    return ops.n == 3 && is_scalar_op(ops.kind[0]) && is_activation(ops.kind[1]) &&
           is_scalar_op(ops.kind[2]);
}

template <class IO>
hipError_t launch_chain_t(const void* x, void* y, int64_t n, const OpList& ops, hipStream_t s) {
    // the fixed-kind kernels serve aligned data; the scalar (unaligned)
    // path keeps the general op loop
    if (chain_is_aaa(ops) && aligned16(x) && aligned16(y))
        return launch_aaa_family<IO>(x, y, n, ops, s);
    return launch_ew<IO>(x, y, n, ChainOp{ops}, s);
}

}  // namespace

hipError_t launch_gelu(const void* x, void* y, int64_t n, Dtype dt, hipStream_t s) {
    return dt == kF32 ? launch_ew<IoF32>(x, y, n, GeluOp{}, s)
                      : launch_ew<IoBF16>(x, y, n, GeluOp{}, s);
}

hipError_t launch_chain(const void* x, void* y, int64_t n, Dtype dt, const OpList& ops,
                        hipStream_t s) {
    return dt == kF32 ? launch_chain_t<IoF32>(x, y, n, ops, s)
                      : launch_chain_t<IoBF16>(x, y, n, ops, s);
}

hipError_t launch_copy(const void* x, void* y, int64_t nbytes, hipStream_t s) {
    if (aligned16(x) && aligned16(y)) {
        const int64_t tile = int64_t(kCopyT) * kCopyU * 16;
        return launch_kernel(reinterpret_cast<const void*>(&copy_vec_kernel<kCopyT, kCopyU, kCopyNT>),
                             grid_for((nbytes + tile - 1) / tile, kCopyT), kCopyT, s,
                             static_cast<const u32x4*>(x), static_cast<u32x4*>(y), nbytes);
    }
    constexpr int kT = 256;
    return launch_kernel(reinterpret_cast<const void*>(&copy_byte_kernel<kT>),
                         grid_for((nbytes + kT * 16 - 1) / (kT * 16), kT), kT, s,
                         static_cast<const uint8_t*>(x), static_cast<uint8_t*>(y), nbytes);
}

}  // namespace fk
