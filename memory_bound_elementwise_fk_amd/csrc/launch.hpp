// launch.hpp -- internal interface between the C ABI layer (api.hip) and the
// kernel launchers (elementwise.hip, softmax.hip). Arguments reaching these
// functions have already been validated; they return a hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fk {

constexpr int kMaxOps = 8;  // equals FK_MAX_OPS of the public header

enum OpKind : int32_t { kOpAdd = 1, kOpMul = 2, kOpGelu = 3 };
enum Dtype : int { kF32 = 0, kBF16 = 1 };

// Op list copied by value into the kernel arguments (no device copy).
struct OpList {
    int32_t n;
    int32_t kind[kMaxOps];
    float scalar[kMaxOps];
};

hipError_t launch_gelu(const void* x, void* y, int64_t n, Dtype dt, hipStream_t s);
hipError_t launch_chain(const void* x, void* y, int64_t n, Dtype dt, const OpList& ops,
                        hipStream_t s);
hipError_t launch_copy(const void* x, void* y, int64_t nbytes, hipStream_t s);

// Softmax over rows; online == true forces the wide-row online path.
hipError_t launch_softmax(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                          int64_t ldy, Dtype dt, bool online, hipStream_t s);
int64_t softmax_onchip_max_cols(Dtype dt);

}  // namespace fk
