// gemm.hip -- launcher of the Linear + GELU kernel (gemm_kernels.hpp).
#include <limits>

#include "gemm_kernels.hpp"
#include "launch.hpp"

namespace fk {
namespace {

// 256 x 256 output tiles, K steps of 64, eight waves of 64 x 128 at two
// waves per SIMD (241 VGPRs, no spills): the fastest of the shapes measured
// on MI355X for an 8192 x 16384 x 4096 product. Four waves of 128 x 128 (one
// per SIMD, 512 registers) were 15-20 % slower: a lone wave leaves the
// matrix cores idle while it waits on LDS and the barrier; 128 x 128 tiles
// (two workgroups per CU) and K steps of 32 were 5-10 % slower.
using LinearShape = GemmShape<256, 256, 64, 64, 128, 2>;
// Same tiles and waves with the operands loaded straight into LDS: K steps
// of 64 in two stages of 64 KiB when K is a multiple of 64 (whole 128-byte
// lines per load; 0.992 against 1.031 ms on 8192 x 16384 x 4096), else K
// steps of 32 in a 4-stage ring loaded three steps ahead when K is a
// multiple of 32 (6 % faster than the register-staged loop); all bitwise the
// same results (same k order).
using LinearDtl64 = DtlShape<256, 256, 64, 128, 2, 2, 64>;
using LinearDtl32 = DtlShape<256, 256, 64, 128, 2, 4, 32>;
static_assert(LinearDtl64::BM == LinearShape::BM && LinearDtl64::BN == LinearShape::BN &&
                  LinearDtl32::BM == LinearShape::BM && LinearDtl32::BN == LinearShape::BN,
              "one tile grid for all kernels");
static_assert(LinearDtl64::kThreads == LinearDtl32::kThreads, "one workgroup size");
constexpr int64_t kMaxWorkItems = int64_t(1) << 31;

}  // namespace

int64_t linear_max_tiles() {
    return kMaxWorkItems / (LinearShape::kThreads > LinearDtl32::kThreads ? LinearShape::kThreads
                                                                         : LinearDtl32::kThreads);
}

// Output tiles of an M x N product (M, N >= 0), saturating at INT64_MAX
// instead of overflowing for sizes the caller will refuse anyway.
int64_t linear_tiles(int64_t M, int64_t N) {
    const int64_t tm = M / LinearShape::BM + (M % LinearShape::BM != 0);
    const int64_t tn = N / LinearShape::BN + (N % LinearShape::BN != 0);
    if (tm != 0 && tn > std::numeric_limits<int64_t>::max() / tm)
        return std::numeric_limits<int64_t>::max();
    return tm * tn;
}

hipError_t launch_linear_gelu(const void* x, const void* w, const void* bias, void* y, int64_t M,
                              int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                              int act, Dtype dt, hipStream_t s) {
    const int64_t tiles = linear_tiles(M, N);
    void* args[] = {const_cast<void**>(&x), const_cast<void**>(&w), const_cast<void**>(&bias), &y,
                    &M, &N, &K, &ldx, &ldw, &ldy, &act};
    const bool f16 = dt == kF16;
    if (K % LinearDtl64::BK == 0) {
        const void* fn =
            f16 ? reinterpret_cast<const void*>(&linear_gelu_dtl_kernel<LinearDtl64, MmaF16>)
                : reinterpret_cast<const void*>(&linear_gelu_dtl_kernel<LinearDtl64, MmaBF16>);
        return hipLaunchKernel(fn, dim3(static_cast<unsigned>(tiles)), dim3(LinearDtl64::kThreads),
                               args, 0, s);
    }
    if (K % LinearDtl32::BK == 0) {
        const void* fn =
            f16 ? reinterpret_cast<const void*>(&linear_gelu_dtl_kernel<LinearDtl32, MmaF16>)
                : reinterpret_cast<const void*>(&linear_gelu_dtl_kernel<LinearDtl32, MmaBF16>);
        return hipLaunchKernel(fn, dim3(static_cast<unsigned>(tiles)), dim3(LinearDtl32::kThreads),
                               args, 0, s);
    }
    const void* fn = f16 ? reinterpret_cast<const void*>(&linear_gelu_kernel<LinearShape, MmaF16>)
                         : reinterpret_cast<const void*>(&linear_gelu_kernel<LinearShape, MmaBF16>);
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(tiles)), dim3(LinearShape::kThreads),
                           args, 0, s);
}

}  // namespace fk
