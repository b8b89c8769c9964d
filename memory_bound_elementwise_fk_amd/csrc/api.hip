// api.hip -- the extern "C" entry points of libfusedops (declared and
// documented in include/fusedops.h). Each validates its arguments on the
// host, before any HIP call, then hands over to a launcher that enqueues one
// kernel on the caller's stream and returns without synchronising.
#include <limits>

#include "fusedops.h"
#include "launch.hpp"

static_assert(FK_MAX_OPS == fk::kMaxOps, "op list size mismatch");
static_assert(int(FK_OP_ADD_SCALAR) == int(fk::kOpAdd) && int(FK_OP_MUL_SCALAR) == int(fk::kOpMul) &&
                  int(FK_OP_GELU_TANH) == int(fk::kOpGelu) && int(FK_OP_RELU) == int(fk::kOpRelu),
              "op kind mismatch");
static_assert(FK_SOFTMAX_SCRATCH_BYTES == fk::kSoftmaxScratchBytes, "scratch size mismatch");
static_assert(int(FK_PATH_ONCHIP) == int(fk::kPathOnChip) &&
                  int(FK_PATH_SPLIT) == int(fk::kPathSplit) &&
                  int(FK_PATH_ONLINE) == int(fk::kPathOnline),
              "softmax path mismatch");
static_assert(int(FK_F32) == int(fk::kF32) && int(FK_BF16) == int(fk::kBF16) &&
                  int(FK_F16) == int(fk::kF16),
              "dtype mismatch");

namespace {

constexpr int64_t kI64Max = std::numeric_limits<int64_t>::max();

// the dtypes of every entry point but Linear and attention (FK_F16 there is
// refused as unsupported, any other value as invalid)
bool dtype_ok(int dtype) { return dtype == FK_F32 || dtype == FK_BF16; }
bool is_f16(int dtype) { return dtype == FK_F16; }
int64_t esize(int dtype) { return dtype == FK_F32 ? 4 : 2; }

// Byte ranges [a, a + na) and [b, b + nb) intersect.
bool ranges_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a);
    const uintptr_t pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + static_cast<uintptr_t>(nb) && pb < pa + static_cast<uintptr_t>(na);
}

int hip_status(hipError_t e) { return e == hipSuccess ? FK_OK : FK_ERR_HIP; }

// Shared checks of the elementwise entry points; sets *nothing_to_do for n == 0.
int check_flat(const void* x, const void* y, int64_t n, int64_t elem_bytes, bool* nothing_to_do) {
    *nothing_to_do = false;
    if (n < 0) return FK_ERR_INVALID_ARG;
    if (n == 0) {
        *nothing_to_do = true;
        return FK_OK;
    }
    if (x == nullptr || y == nullptr) return FK_ERR_INVALID_ARG;
    if (n > kI64Max / elem_bytes) return FK_ERR_UNSUPPORTED;
    const int64_t bytes = n * elem_bytes;
    if (x != y && ranges_overlap(x, bytes, y, bytes)) return FK_ERR_OVERLAP;
    return FK_OK;
}

int check_rows(const void* x, const void* y, int64_t rows, int64_t cols, int64_t ldx,
               int64_t ldy, int dtype, bool* nothing_to_do) {
    *nothing_to_do = false;
    if (is_f16(dtype)) return FK_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return FK_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0) return FK_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) {
        *nothing_to_do = true;
        return FK_OK;
    }
    if (x == nullptr || y == nullptr) return FK_ERR_INVALID_ARG;
    if (ldx < cols || ldy < cols) return FK_ERR_INVALID_ARG;
    const int64_t es = esize(dtype);
    // extent in elements of each operand: (rows - 1) * ld + cols, in bytes
    if (rows - 1 > (kI64Max / es - cols) / ldx || rows - 1 > (kI64Max / es - cols) / ldy)
        return FK_ERR_UNSUPPORTED;
    const int64_t bx = ((rows - 1) * ldx + cols) * es;
    const int64_t by = ((rows - 1) * ldy + cols) * es;
    if (x == y) {
        if (ldx != ldy) return FK_ERR_OVERLAP;
    } else if (ranges_overlap(x, bx, y, by)) {
        return FK_ERR_OVERLAP;
    }
    return FK_OK;
}

int softmax_launch(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy,
                   int dtype, bool online, void* ws, int64_t ws_bytes, void* stream) {
    return hip_status(fk::launch_softmax(x, y, rows, cols, ldx, ldy, static_cast<fk::Dtype>(dtype),
                                         online, ws, ws_bytes, static_cast<hipStream_t>(stream)));
}

// Validation of fk_softmax_rows_ws's workspace, for a call that passed
// check_rows with work to do: FK_OK when the split path does not apply or
// the workspace serves it.
int check_workspace(const void* x, const void* y, int64_t rows, int64_t cols, int64_t ldx,
                    int64_t ldy, int dtype, const void* workspace, int64_t workspace_bytes) {
    const int64_t need = fk::softmax_workspace_bytes(rows, cols, static_cast<fk::Dtype>(dtype));
    if (need == 0 || x == y) return FK_OK;  // no split path: the workspace is not used
    if (workspace == nullptr || workspace_bytes < need) return FK_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(workspace) & 7u) != 0) return FK_ERR_INVALID_ARG;
    const int64_t es = esize(dtype);
    if (ranges_overlap(workspace, need, x, ((rows - 1) * ldx + cols) * es) ||
        ranges_overlap(workspace, need, y, ((rows - 1) * ldy + cols) * es))
        return FK_ERR_OVERLAP;
    return FK_OK;
}

}  // namespace

extern "C" {

int fk_gelu_tanh(const void* x, void* y, int64_t n, int dtype, void* stream) {
    if (is_f16(dtype)) return FK_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return FK_ERR_INVALID_ARG;
    bool skip = false;
    const int st = check_flat(x, y, n, esize(dtype), &skip);
    if (st != FK_OK || skip) return st;
    return hip_status(
        fk::launch_gelu(x, y, n, static_cast<fk::Dtype>(dtype), static_cast<hipStream_t>(stream)));
}

int fk_elementwise_chain(const void* x, void* y, int64_t n, int dtype, const fk_op* ops,
                         int n_ops, void* stream) {
    if (is_f16(dtype)) return FK_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return FK_ERR_INVALID_ARG;
    if (ops == nullptr || n_ops < 1 || n_ops > FK_MAX_OPS) return FK_ERR_INVALID_ARG;
    fk::OpList list{};
    list.n = n_ops;
    for (int i = 0; i < n_ops; ++i) {
        const int32_t k = ops[i].kind;
        if (k != FK_OP_ADD_SCALAR && k != FK_OP_MUL_SCALAR && k != FK_OP_GELU_TANH &&
            k != FK_OP_RELU)
            return FK_ERR_INVALID_ARG;
        list.kind[i] = k;
        list.scalar[i] = ops[i].scalar;
    }
    bool skip = false;
    const int st = check_flat(x, y, n, esize(dtype), &skip);
    if (st != FK_OK || skip) return st;
    return hip_status(fk::launch_chain(x, y, n, static_cast<fk::Dtype>(dtype), list,
                                       static_cast<hipStream_t>(stream)));
}

int fk_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy,
                    int dtype, void* stream) {
    bool skip = false;
    const int st = check_rows(x, y, rows, cols, ldx, ldy, dtype, &skip);
    if (st != FK_OK || skip) return st;
    return softmax_launch(x, y, rows, cols, ldx, ldy, dtype, false, nullptr, 0, stream);
}

int fk_softmax_rows_ws(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                       int64_t ldy, int dtype, void* workspace, int64_t workspace_bytes,
                       void* stream) {
    bool skip = false;
    int st = check_rows(x, y, rows, cols, ldx, ldy, dtype, &skip);
    if (st != FK_OK) return st;
    if (workspace_bytes < 0) return FK_ERR_INVALID_ARG;
    if (skip) return FK_OK;
    st = check_workspace(x, y, rows, cols, ldx, ldy, dtype, workspace, workspace_bytes);
    if (st != FK_OK) return st;
    return softmax_launch(x, y, rows, cols, ldx, ldy, dtype, false, workspace, workspace_bytes,
                          stream);
}

int fk_softmax_rows_noalloc(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                            int64_t ldy, int dtype, void* stream) {
    bool skip = false;
    const int st = check_rows(x, y, rows, cols, ldx, ldy, dtype, &skip);
    if (st != FK_OK || skip) return st;
    const int64_t need = x == y ? 0 : fk::softmax_workspace_bytes(rows, cols, static_cast<fk::Dtype>(dtype));
    if (need > fk::kSoftmaxScratchBytes) return FK_ERR_UNSUPPORTED;
    void* ws = nullptr;
    if (need > 0) {
        const hipError_t e = fk::softmax_scratch(&ws);
        if (e != hipSuccess) return FK_ERR_HIP;
    }
    return softmax_launch(x, y, rows, cols, ldx, ldy, dtype, false, ws, need, stream);
}

int fk_softmax_rows_path(const void* x, const void* y, int64_t rows, int64_t cols, int64_t ldx,
                         int64_t ldy, int dtype, int64_t workspace_bytes) {
    bool skip = false;
    int st = check_rows(x, y, rows, cols, ldx, ldy, dtype, &skip);
    if (st != FK_OK) return st;
    if (workspace_bytes < 0) return FK_ERR_INVALID_ARG;
    if (skip) return FK_PATH_NONE;
    return fk::softmax_path(rows, cols, static_cast<fk::Dtype>(dtype), x == y, false,
                            workspace_bytes);
}

int64_t fk_softmax_workspace_bytes(int64_t rows, int64_t cols, int dtype) {
    if (is_f16(dtype)) return FK_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype) || rows < 0 || cols < 0) return FK_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return 0;
    return fk::softmax_workspace_bytes(rows, cols, static_cast<fk::Dtype>(dtype));
}

int64_t fk_set_split_wait_limit(int64_t polls) {
    if (polls < 0) return FK_ERR_INVALID_ARG;
    return fk::set_split_wait_limit(polls);
}

int fk_softmax_rows_online(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                           int64_t ldy, int dtype, void* stream) {
    bool skip = false;
    const int st = check_rows(x, y, rows, cols, ldx, ldy, dtype, &skip);
    if (st != FK_OK || skip) return st;
    return softmax_launch(x, y, rows, cols, ldx, ldy, dtype, true, nullptr, 0, stream);
}

int fk_layernorm_rows(const void* x, void* y, int64_t rows, int64_t cols, int64_t ldx,
                      int64_t ldy, const void* gamma, const void* beta, float eps, int fuse_gelu,
                      int dtype, void* stream) {
    bool skip = false;
    const int st = check_rows(x, y, rows, cols, ldx, ldy, dtype, &skip);
    if (st != FK_OK) return st;
    if (!(eps >= 0.0f) || eps == std::numeric_limits<float>::infinity()) return FK_ERR_INVALID_ARG;
    if (fuse_gelu != 0 && fuse_gelu != 1) return FK_ERR_INVALID_ARG;
    if (skip) return FK_OK;
    if (cols > fk::layernorm_max_cols(static_cast<fk::Dtype>(dtype))) return FK_ERR_UNSUPPORTED;
    const int64_t es = esize(dtype);
    const int64_t by = ((rows - 1) * ldy + cols) * es;
    // gamma and beta are read by every row while y is written
    if ((gamma != nullptr && ranges_overlap(gamma, cols * es, y, by)) ||
        (beta != nullptr && ranges_overlap(beta, cols * es, y, by)))
        return FK_ERR_OVERLAP;
    return hip_status(fk::launch_layernorm(x, y, rows, cols, ldx, ldy, gamma, beta, eps, fuse_gelu,
                                           static_cast<fk::Dtype>(dtype),
                                           static_cast<hipStream_t>(stream)));
}

int fk_gelu_tanh_backward(const void* x, const void* dy, void* dx, int64_t n, int dtype,
                          void* stream) {
    if (is_f16(dtype)) return FK_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return FK_ERR_INVALID_ARG;
    bool skip = false;
    int st = check_flat(x, dx, n, esize(dtype), &skip);  // also: dx == x or disjoint
    if (st != FK_OK || skip) return st;
    st = check_flat(dy, dx, n, esize(dtype), &skip);      // dx == dy or disjoint
    if (st != FK_OK) return st;
    return hip_status(fk::launch_gelu_backward(x, dy, dx, n, static_cast<fk::Dtype>(dtype),
                                               static_cast<hipStream_t>(stream)));
}

int fk_softmax_rows_backward(const void* y, const void* dy, void* dx, int64_t rows, int64_t cols,
                             int64_t ldy, int64_t lddy, int64_t lddx, int dtype, void* stream) {
    bool skip = false;
    int st = check_rows(y, dx, rows, cols, ldy, lddx, dtype, &skip);
    if (st != FK_OK) return st;
    st = check_rows(dy, dx, rows, cols, lddy, lddx, dtype, &skip);
    if (st != FK_OK || skip) return st;
    if (cols > fk::softmax_backward_max_cols(static_cast<fk::Dtype>(dtype)))
        return FK_ERR_UNSUPPORTED;
    return hip_status(fk::launch_softmax_backward(y, dy, dx, rows, cols, ldy, lddy, lddx,
                                                  static_cast<fk::Dtype>(dtype),
                                                  static_cast<hipStream_t>(stream)));
}

int64_t fk_softmax_backward_max_cols(int dtype) {
    if (is_f16(dtype)) return FK_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return FK_ERR_INVALID_ARG;
    return fk::softmax_backward_max_cols(static_cast<fk::Dtype>(dtype));
}

int fk_linear_gelu(const void* x, const void* w, const void* bias, void* y, int64_t M, int64_t N,
                   int64_t K, int64_t ldx, int64_t ldw, int64_t ldy, int act, int dtype,
                   void* stream) {
    if (!dtype_ok(dtype) && !is_f16(dtype)) return FK_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0) return FK_ERR_INVALID_ARG;
    if (act != FK_ACT_NONE && act != FK_ACT_GELU_TANH && act != FK_ACT_RELU)
        return FK_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return FK_OK;
    if (y == nullptr || (K > 0 && (x == nullptr || w == nullptr))) return FK_ERR_INVALID_ARG;
    if (ldy < N || (K > 0 && (ldx < K || ldw < K))) return FK_ERR_INVALID_ARG;
    if (dtype == FK_F32) return FK_ERR_UNSUPPORTED;
    // x and w are read only when K > 0 (K == 0 gives GELU(bias))
    // the kernels count K steps (of 32 or more) in 32 bits
    if (K >= (int64_t(1) << 36)) return FK_ERR_UNSUPPORTED;
    if (K > 0 && (K % 8 != 0 || ldx % 8 != 0 || ldw % 8 != 0 ||
                  ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w)) & 15u) != 0))
        return FK_ERR_UNSUPPORTED;
    if (fk::linear_tiles(M, N) > fk::linear_max_tiles()) return FK_ERR_UNSUPPORTED;
    if (M - 1 > (kI64Max / 2 - N) / ldy || (K > 0 && (M - 1 > (kI64Max / 2 - K) / ldx ||
                                                     N - 1 > (kI64Max / 2 - K) / ldw)))
        return FK_ERR_UNSUPPORTED;
    const int64_t by = ((M - 1) * ldy + N) * 2;
    if (K > 0 && (ranges_overlap(y, by, x, ((M - 1) * ldx + K) * 2) ||
                  ranges_overlap(y, by, w, ((N - 1) * ldw + K) * 2)))
        return FK_ERR_OVERLAP;
    if (bias != nullptr && ranges_overlap(y, by, bias, N * 2)) return FK_ERR_OVERLAP;
    return hip_status(fk::launch_linear_gelu(x, w, bias, y, M, N, K, ldx, ldw, ldy, act,
                                             static_cast<fk::Dtype>(dtype),
                                             static_cast<hipStream_t>(stream)));
}

int fk_attention_fwd(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
                     int64_t T, int64_t d, const int64_t* strides, int causal, int dtype,
                     void* stream) {
    if ((!dtype_ok(dtype) && !is_f16(dtype)) || B < 0 || H < 0 || T < 0 || d < 1)
        return FK_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FK_ERR_INVALID_ARG;
    if (strides == nullptr) return FK_ERR_INVALID_ARG;
    if (B == 0 || H == 0 || T == 0) return FK_OK;
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FK_ERR_INVALID_ARG;
    for (int i = 0; i < 12; ++i)
        if (strides[i] < 0) return FK_ERR_INVALID_ARG;
    for (int t = 0; t < 4; ++t)
        if (strides[3 * t + 2] < d) return FK_ERR_INVALID_ARG;  // rows of d contiguous values
    if (dtype == FK_F32 || d != fk::attention_head_dim()) return FK_ERR_UNSUPPORTED;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                           reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o);
    if ((addr & 15u) != 0) return FK_ERR_UNSUPPORTED;
    for (int i = 0; i < 12; ++i)
        if (strides[i] % 8 != 0) return FK_ERR_UNSUPPORTED;
    // at most one workgroup per 128 queries of one head, at most 2^23 of them
    if (B > (int64_t(1) << 31) / H || T > (int64_t(1) << 40)) return FK_ERR_UNSUPPORTED;
    if (B * H > fk::kAttnMaxWorkgroups / fk::attention_workgroups(1, 1, T))
        return FK_ERR_UNSUPPORTED;
    // extent in bytes of each operand: the last element's offset + 1
    int64_t ext[4];
    for (int t = 0; t < 4; ++t) {
        const int64_t* st = strides + 3 * t;
        if ((B - 1) > kI64Max / 8 / (st[0] + 1) || (H - 1) > kI64Max / 8 / (st[1] + 1) ||
            (T - 1) > kI64Max / 8 / (st[2] + 1))
            return FK_ERR_UNSUPPORTED;
        ext[t] = ((B - 1) * st[0] + (H - 1) * st[1] + (T - 1) * st[2] + d) * 2;
    }
    if (ranges_overlap(o, ext[3], q, ext[0]) || ranges_overlap(o, ext[3], k, ext[1]) ||
        ranges_overlap(o, ext[3], v, ext[2]))
        return FK_ERR_OVERLAP;
    return hip_status(fk::launch_attention_fwd(q, k, v, o, B, H, T, strides, causal,
                                               static_cast<fk::Dtype>(dtype),
                                               static_cast<hipStream_t>(stream)));
}

int64_t fk_layernorm_max_cols(int dtype) {
    if (is_f16(dtype)) return FK_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return FK_ERR_INVALID_ARG;
    return fk::layernorm_max_cols(static_cast<fk::Dtype>(dtype));
}

int64_t fk_softmax_onchip_max_cols(int dtype) {
    if (is_f16(dtype)) return FK_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return FK_ERR_INVALID_ARG;
    return fk::softmax_onchip_max_cols(static_cast<fk::Dtype>(dtype));
}

int fk_copy(const void* x, void* y, int64_t nbytes, void* stream) {
    bool skip = false;
    const int st = check_flat(x, y, nbytes, 1, &skip);
    if (st != FK_OK || skip) return st;
    return hip_status(fk::launch_copy(x, y, nbytes, static_cast<hipStream_t>(stream)));
}

const char* fk_status_string(int status) {
    switch (status) {
        case FK_OK: return "ok";
        case FK_ERR_INVALID_ARG: return "invalid argument";
        case FK_ERR_UNSUPPORTED: return "unsupported size";
        case FK_ERR_OVERLAP: return "input and output overlap without being equal";
        case FK_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

}  // extern "C"
