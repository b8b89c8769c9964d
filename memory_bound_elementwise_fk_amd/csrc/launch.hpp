// launch.hpp -- internal interface between the C ABI layer (api.hip) and the
// kernel launchers (elementwise.hip, softmax.hip, ...). Arguments reaching these
// functions have already been validated; they return a hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace fk {

// Compute units of the current device (queried once per device; 0 if the
// query fails).
inline int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

constexpr int kMaxOps = 8;  // equals FK_MAX_OPS of the public header

enum OpKind : int32_t { kOpAdd = 1, kOpMul = 2, kOpGelu = 3, kOpRelu = 4 };
enum Dtype : int { kF32 = 0, kBF16 = 1, kF16 = 2 };  // kF16: Linear and attention only

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

// Softmax over rows. Path: rows up to softmax_onchip_max_cols(dt) columns
// run the single-pass kernel; wider rows run the split kernel when `ws`
// holds at least softmax_workspace_bytes() bytes (any contents) and y != x,
// else the online two-pass kernel. online == true forces the online kernel.
enum SoftmaxPath : int { kPathOnChip = 1, kPathSplit = 2, kPathOnline = 3 };
hipError_t launch_softmax(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                          int64_t ldy, Dtype dt, bool online, void* ws, int64_t ws_bytes,
                          hipStream_t s);
// The path launch_softmax takes for these arguments (rows, cols >= 1).
SoftmaxPath softmax_path(int64_t rows, int64_t cols, Dtype dt, bool in_place, bool online,
                         int64_t ws_bytes);
int64_t softmax_onchip_max_cols(Dtype dt);
// Workspace the split path needs for this shape; 0 if it does not apply.
int64_t softmax_workspace_bytes(int64_t rows, int64_t cols, Dtype dt);
// The library's static split-path scratch on the current device (address
// looked up once per device); kSoftmaxScratchBytes bytes, any contents.
constexpr int64_t kSoftmaxScratchBytes = int64_t(1) << 20;
hipError_t softmax_scratch(void** ptr);
// Bound on the polls of a split-kernel block waiting for its row's other
// slices; past it the block computes the row statistics itself.
int64_t split_wait_limit();
int64_t set_split_wait_limit(int64_t polls);

// Fused LayerNorm (+ optional tanh-GELU) over rows of at most
// layernorm_max_cols(dt) columns; gamma / beta may be null.
hipError_t launch_layernorm(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t ldy, const void* gamma, const void* beta, float eps, int gelu,
                            Dtype dt, hipStream_t s);
int64_t layernorm_max_cols(Dtype dt);

// Backward kernels: dx = dy * GELU'(x) elementwise; softmax backward
// dx = y (dy - sum y dy) over rows of at most softmax_backward_max_cols(dt).
hipError_t launch_gelu_backward(const void* x, const void* dy, void* dx, int64_t n, Dtype dt,
                                hipStream_t s);
hipError_t launch_softmax_backward(const void* y, const void* dy, void* dx, int64_t rows,
                                   int64_t cols, int64_t ldy, int64_t lddy, int64_t lddx,
                                   Dtype dt, hipStream_t s);
int64_t softmax_backward_max_cols(Dtype dt);

// Y = act(X W^T + b), act 0 none, 1 tanh-GELU, 2 ReLU (bf16 or fp16, fp32
// accumulation on MFMA); arguments
// validated by the caller: K, ldx, ldw multiples of 8, X and W 16-byte
// aligned, linear_tiles(M, N) <= linear_max_tiles().
hipError_t launch_linear_gelu(const void* x, const void* w, const void* bias, void* y, int64_t M,
                              int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                              int act, Dtype dt, hipStream_t s);
int64_t linear_tiles(int64_t M, int64_t N);
int64_t linear_max_tiles();

// FlashAttention forward, bf16 or fp16, head dimension attention_head_dim();
// strides[12] = (batch, head, row) strides of q, k, v, o in elements.
hipError_t launch_attention_fwd(const void* q, const void* k, const void* v, void* o, int64_t B,
                                int64_t H, int64_t T, const int64_t* strides, int causal, Dtype dt,
                                hipStream_t s);
int64_t attention_head_dim();
// workgroups of a launch in 4-wave workgroups, the most the launcher uses:
// ceil(T / 128) * B * H (caller keeps it <= 2^23 so the grid stays below
// 2^31 work-items); B * H must not overflow
int64_t attention_workgroups(int64_t B, int64_t H, int64_t T);
constexpr int64_t kAttnMaxWorkgroups = int64_t(1) << 23;

}  // namespace fk
