// gemm.hip -- launcher of the Linear + GELU kernel (gemm_kernels.hpp).
#include "gemm_kernels.hpp"
#include "launch.hpp"

namespace fk {
namespace {

// 256 x 256 output tiles, K steps of 64, four waves of 128 x 128: the
// fastest of the shapes measured on MI355X for an 8192 x 16384 x 4096
// product (128 x 128, 128 x 256, 256 x 128 tiles and K steps of 32 were
// 0-25 % slower).
using LinearShape = GemmShape<256, 256, 64, 128, 128>;
constexpr int64_t kMaxWorkItems = int64_t(1) << 31;

}  // namespace

int64_t linear_max_tiles() { return kMaxWorkItems / LinearShape::kThreads; }

int64_t linear_tiles(int64_t M, int64_t N) {
    return ((M + LinearShape::BM - 1) / LinearShape::BM) * ((N + LinearShape::BN - 1) / LinearShape::BN);
}

hipError_t launch_linear_gelu(const void* x, const void* w, const void* bias, void* y, int64_t M,
                              int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                              int gelu, hipStream_t s) {
    const int64_t tiles = linear_tiles(M, N);
    void* args[] = {const_cast<void**>(&x), const_cast<void**>(&w), const_cast<void**>(&bias), &y,
                    &M, &N, &K, &ldx, &ldw, &ldy, &gelu};
    return hipLaunchKernel(reinterpret_cast<const void*>(&linear_gelu_kernel<LinearShape>),
                           dim3(static_cast<unsigned>(tiles)), dim3(LinearShape::kThreads), args, 0,
                           s);
}

}  // namespace fk
