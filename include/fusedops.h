/*
 * fusedops.h -- C ABI of libfusedops: fused memory-bound kernels for AMD
 * Instinct MI355X (gfx950), each reading every element from HBM once and
 * writing it once.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: x and y are DEVICE pointers owned by the caller. The library
 *   never allocates, frees, copies or synchronises device memory: the one
 *   scratch buffer a kernel uses (the split softmax's partial statistics)
 *   is the caller's, passed to fk_softmax_rows_ws. Op lists (fk_op arrays)
 *   are HOST pointers, read before the call returns.
 * Stream: a hipStream_t passed as void*; NULL is the null stream. Work is
 *   enqueued on it and the call returns without waiting (launches are
 *   asynchronous, as the profiling notes on the pages stress: the host runs
 *   ahead of the device until it synchronises).
 * dtype: FK_F32 (IEEE binary32) or FK_BF16 (bfloat16, the upper half of a
 *   binary32); FK_F16 (IEEE binary16) for fk_linear_gelu and fk_attention_fwd
 *   only, every other entry point returns FK_ERR_UNSUPPORTED for it. Input and output share
 *   the dtype. All arithmetic is fp32; bf16 and fp16 outputs are rounded to
 *   nearest, ties to even; NaN stays NaN.
 * Sizes: element counts and strides are in ELEMENTS (not bytes), int64_t.
 * Aliasing: y == x (exactly in place, and for row ops also ldy == ldx) is
 *   allowed: every element is read before the same lane writes it. Any
 *   other overlap of the input and output byte ranges is FK_ERR_OVERLAP.
 * Alignment: any element-aligned pointer is accepted; 16-byte aligned data
 *   takes the 128-bit vector path, other data a scalar path.
 * Empty work (n == 0, rows == 0 or cols == 0) returns FK_OK and launches
 *   nothing; pointers may then be NULL.
 * Errors: invalid arguments return a negative fk_status BEFORE any HIP call
 *   and nothing is launched. A failed launch returns FK_ERR_HIP.
 * Threads: entry points keep no per-call state and may be called
 *   concurrently; the one process-wide setting is the wait bound of
 *   fk_set_split_wait_limit.
 */
#ifndef FUSEDOPS_H
#define FUSEDOPS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FK_F32 = 0, FK_BF16 = 1, FK_F16 = 2 } fk_dtype;

typedef enum {
    FK_OK = 0,
    FK_ERR_INVALID_ARG = -1, /* null pointer with work to do, negative size,
                                stride < cols, unknown dtype, bad op list   */
    FK_ERR_UNSUPPORTED = -2, /* valid but not handled here: a size beyond
                                what one launch can address, a row wider
                                than the entry point's capacity, FK_F16
                                outside Linear and attention, an attention
                                head dimension other than 128               */
    FK_ERR_OVERLAP = -3,     /* input and output overlap without being equal */
    FK_ERR_HIP = -4          /* the HIP runtime reported an error           */
} fk_status;

/* Elementwise op kinds of a fused chain. */
typedef enum {
    FK_OP_ADD_SCALAR = 1, /* v = v + scalar               */
    FK_OP_MUL_SCALAR = 2, /* v = v * scalar               */
    FK_OP_GELU_TANH = 3,  /* v = tanh-GELU(v); scalar ignored */
    FK_OP_RELU = 4        /* v = v > 0 ? v : +0, NaN kept; scalar ignored */
} fk_op_kind;

typedef struct {
    int32_t kind;  /* an fk_op_kind */
    float scalar;  /* operand of ADD / MUL */
} fk_op;

#define FK_MAX_OPS 8

/*
 * tanh-GELU, y[i] = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) for
 * i in [0, n), as defined in the "CS336 lecture 6" notes (kyc001.github.io),
 * section 4.2 "Case: GELU"; fused so that x is read once and y written once
 * (section 4.1 of the same notes).
 * Evaluated as the identical real function x / (1 + 2^t),
 * t = x (A + B x^2), A = -2 sqrt(2/pi) log2(e), B = 0.044715 A, which does
 * not cancel for negative x. Relative error <= 1e-5 for x >= -9 (fp32 out);
 * GELU(+-0) = +-0, GELU(+inf) = +inf, GELU(-inf) = -0, GELU(NaN) = NaN.
 * x, y: device arrays of n elements of dtype.
 */
int fk_gelu_tanh(const void* x, void* y, int64_t n, int dtype, void* stream);

/*
 * Fused elementwise chain: for every i in [0, n), v = x[i]; then each op of
 * ops[0 .. n_ops) in order; y[i] = v. One HBM read and one write per
 * element instead of one per op ("Lecture 6: GPU Kernels and Triton",
 * cs336.sjfarmltd.com, section 1.1: three consecutive elementwise ops over
 * 32 MB move 192 MB unfused and 64 MB fused). Every intermediate is
 * rounded to fp32, so the fused result equals running each op as its own
 * fp32 kernel (and is bitwise equal to it for ADD and MUL).
 * ops: host array of n_ops in [1, FK_MAX_OPS] entries, copied by value into
 * the launch. Unknown kinds are FK_ERR_INVALID_ARG.
 */
int fk_elementwise_chain(const void* x, void* y, int64_t n, int dtype,
                         const fk_op* ops, int n_ops, void* stream);

/*
 * Row softmax: for each row r in [0, rows), with x_r = x + r*ldx and
 * y_r = y + r*ldy: m = max_j x_r[j]; s = sum_j exp(x_r[j] - m);
 * y_r[j] = exp(x_r[j] - m) / s for j in [0, cols) ("CS336 lecture 6" notes,
 * section 5.2: one block per row, max, exponentials and their sum,
 * normalise and write back). Entries past cols in a row (the stride
 * padding) are neither read nor written. fp32 accumulation.
 * Paths (fk_softmax_rows_path tells which one a call takes):
 *  - FK_PATH_ONCHIP, rows up to fk_softmax_onchip_max_cols(dtype) columns:
 *    one workgroup (or one wave) per row, the row held in registers; each
 *    element is read from HBM once and written once;
 *  - FK_PATH_ONLINE, wider rows: the online two-pass kernel of
 *    fk_softmax_rows_online (one workgroup per row; the part of the row that
 *    does not stay on chip is read twice).
 * fk_softmax_rows_ws reads wide rows once instead (FK_PATH_SPLIT), with a
 * caller workspace. Allocates nothing.
 * A row with NaN or +inf, or only -inf, comes out all NaN (the formula).
 * ldx, ldy: row strides in elements, >= cols.
 */
int fk_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols,
                    int64_t ldx, int64_t ldy, int dtype, void* stream);

/*
 * fk_softmax_rows with a caller workspace for rows wider than on-chip
 * capacity (FK_PATH_SPLIT): each row is cut into slices of 8192 columns
 * (at most 64), one workgroup per slice holding it in registers, so every
 * element is read from HBM once and written once. The slices of a row
 * exchange partial (max, sum) pairs through the workspace and merge them
 * with the online softmax rule of "Lecture 6: GPU Kernels and Triton",
 * section 7.2.
 * workspace: DEVICE memory of at least fk_softmax_workspace_bytes(rows,
 *   cols, dtype) bytes, 8-byte aligned, with ANY contents: every slot word
 *   carries a tag drawn afresh for each call, so zeros, a previous call's
 *   partials or garbage are never read as this call's. Nothing needs
 *   clearing before or after a call. Calls sharing a workspace should be
 *   ordered (one stream): overlapping ones overwrite each other's slots,
 *   which sends the affected workgroups to their bounded-wait fallback
 *   (still correct, slower; see fk_set_split_wait_limit).
 * The workspace is not used -- and may be NULL -- when that size is 0, and
 * in place (y == x), where wide rows take FK_PATH_ONLINE: a split
 * workgroup's fallback re-reads the whole row, which other slices may
 * already have overwritten.
 * Errors: FK_ERR_INVALID_ARG for a missing, misaligned or too small
 * workspace (when it is used) or workspace_bytes < 0; FK_ERR_OVERLAP if it
 * overlaps x or y.
 */
int fk_softmax_rows_ws(const void* x, void* y, int64_t rows, int64_t cols,
                       int64_t ldx, int64_t ldy, int dtype, void* workspace,
                       int64_t workspace_bytes, void* stream);

/*
 * Bytes of workspace the split path needs for rows x cols of dtype:
 * rows * slices * 16 (two 8-byte words per slice), slices = ceil(cols /
 * 8192); 0 when the rows fit on chip or the split path does not apply
 * (more than 64 slices). FK_ERR_INVALID_ARG for negative sizes or an
 * unknown dtype. Pure host query.
 */
int64_t fk_softmax_workspace_bytes(int64_t rows, int64_t cols, int dtype);

/*
 * fk_softmax_rows_ws for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the split path's workspace is the library's own static device
 * array of FK_SOFTMAX_SCRATCH_BYTES bytes (one per GPU, held until the
 * process ends) instead of a caller buffer. The call allocates and frees
 * nothing. Same paths and results as fk_softmax_rows_ws with a large enough
 * workspace.
 * Limit: shapes whose split path needs more than FK_SOFTMAX_SCRATCH_BYTES
 * (fk_softmax_workspace_bytes(rows, cols, dtype) > 1 MiB, e.g. more than
 * 65536 rows x slices) return FK_ERR_UNSUPPORTED before any HIP call.
 * Nothing in the array needs clearing (every slot word carries a per-call
 * tag). Calls that overlap on one GPU (different streams) share the array
 * and race for its slots: a workgroup whose partials were overwritten waits
 * out its bound (fk_set_split_wait_limit) and computes its row's statistics
 * by streaming the row -- correct, but slow. Order such calls on one stream.
 * FK_ERR_HIP if the array's device address cannot be obtained.
 */
#define FK_SOFTMAX_SCRATCH_BYTES (1 << 20)
int fk_softmax_rows_noalloc(const void* x, void* y, int64_t rows, int64_t cols,
                            int64_t ldx, int64_t ldy, int dtype, void* stream);

/* Kernel paths of the row softmax. */
typedef enum {
    FK_PATH_NONE = 0,   /* empty work: nothing launched              */
    FK_PATH_ONCHIP = 1, /* one row per workgroup, held in registers  */
    FK_PATH_SPLIT = 2,  /* slices of a row over several workgroups   */
    FK_PATH_ONLINE = 3  /* one workgroup streams the row twice       */
} fk_softmax_path;

/*
 * The path (an fk_softmax_path) that fk_softmax_rows_ws takes for these
 * arguments with a workspace of workspace_bytes bytes; workspace_bytes = 0
 * gives the path of fk_softmax_rows. Arguments that call would reject
 * return its negative fk_status. Pure host query: x and y are compared
 * (y == x selects the in-place path), never dereferenced.
 */
int fk_softmax_rows_path(const void* x, const void* y, int64_t rows,
                         int64_t cols, int64_t ldx, int64_t ldy, int dtype,
                         int64_t workspace_bytes);

/*
 * Bound on the polls (each followed by a short sleep) that a split-path
 * workgroup spends waiting for the other slices of its row. Past it the
 * workgroup computes the row's max and sum by streaming the whole row
 * itself, so the kernel ends and stays correct whatever the scheduling.
 * Default 2^20. Returns the previous bound, or FK_ERR_INVALID_ARG for
 * polls < 0. Process-wide; for tests and diagnostics (0: every split
 * workgroup polls once, so all but those that find every partial already
 * published take the streamed statistics).
 */
int64_t fk_set_split_wait_limit(int64_t polls);

/*
 * Same result as fk_softmax_rows, always through the wide-row online path:
 * pass 1 streams the row and keeps a running max m and a running sum l,
 * rescaling l by exp(m_old - m_new) whenever the max grows ("Lecture 6:
 * GPU Kernels and Triton", section 7.2 "Online Softmax", without the
 * attention accumulator); partial (m, l) pairs merge by the same rule;
 * pass 2 writes exp(x - m) / l. One workgroup per row. For 16-byte aligned
 * rows of < 2^31 bytes the first 131072 fp32 or 262144 bf16 columns (whole
 * 8192-column chunks, 512 KiB) stay on chip -- in VGPRs and LDS -- between
 * the passes, so only the rest of the row is read twice; other rows are
 * read twice. Any cols >= 1.
 */
int fk_softmax_rows_online(const void* x, void* y, int64_t rows, int64_t cols,
                           int64_t ldx, int64_t ldy, int dtype, void* stream);

/*
 * Fused LayerNorm over each row, optionally followed by tanh-GELU: with
 * x_r, y_r as for fk_softmax_rows, mu = mean_j x_r[j],
 * var = mean_j (x_r[j] - mu)^2 (biased),
 * t_j = (x_r[j] - mu) / sqrt(var + eps) * gamma[j] + beta[j],
 * y_r[j] = fuse_gelu ? GELU(t_j) : t_j. LayerNorm is the first stage of the
 * LayerNorm -> Linear -> GELU fusion example of "Lecture 6: GPU Kernels and
 * Triton", section 6.1 (the page gives no formula; this is the standard
 * definition). One read of x and one write of y per element, fp32
 * statistics (corrected two-pass over the row held in registers).
 * gamma, beta: DEVICE arrays of cols elements of dtype, or NULL (1 and 0);
 * they must not overlap y (FK_ERR_OVERLAP). eps: finite, >= 0.
 * fuse_gelu: 0 or 1. Rows wider than fk_layernorm_max_cols(dtype) are
 * FK_ERR_UNSUPPORTED. In place (y == x, same stride) is allowed.
 */
int fk_layernorm_rows(const void* x, void* y, int64_t rows, int64_t cols,
                      int64_t ldx, int64_t ldy, const void* gamma,
                      const void* beta, float eps, int fuse_gelu, int dtype,
                      void* stream);

/* Widest row fk_layernorm_rows accepts for dtype (32768 fp32, 65536 bf16),
 * or FK_ERR_INVALID_ARG for an unknown dtype. Pure host query. */
int64_t fk_layernorm_max_cols(int dtype);

/*
 * GELU backward: dx[i] = dy[i] * GELU'(x[i]) for i in [0, n), GELU' the
 * derivative of the tanh-GELU of fk_gelu_tanh (the pages print no backward
 * formula; this is the derivative of their forward definition):
 * GELU'(x) = s + 2 sqrt(2/pi) x (1 + 3 * 0.044715 x^2) s (1 - s),
 * s = 1 / (1 + exp(-2u)). Two reads and one write per element.
 * GELU'(+inf) = 1, GELU'(-inf) = 0, NaN stays NaN. x, dy, dx: device arrays
 * of n elements of dtype; dx may be x or dy exactly, any other overlap with
 * them is FK_ERR_OVERLAP (x and dy may overlap each other).
 */
int fk_gelu_tanh_backward(const void* x, const void* dy, void* dx, int64_t n,
                          int dtype, void* stream);

/*
 * Row softmax backward: for each row, with y the softmax output and dy the
 * incoming gradient, dx_j = y_j (dy_j - sum_k y_k dy_k) (the product of the
 * softmax Jacobian with dy; derived from the forward definition of
 * fk_softmax_rows). Row strides ldy, lddy, lddx in elements, >= cols. The row
 * is held in registers: one read of y and dy, one write of dx per element.
 * dx may be y or dy exactly (same stride); other overlaps are
 * FK_ERR_OVERLAP. Rows wider than fk_softmax_backward_max_cols(dtype) are
 * FK_ERR_UNSUPPORTED.
 */
int fk_softmax_rows_backward(const void* y, const void* dy, void* dx,
                             int64_t rows, int64_t cols, int64_t ldy,
                             int64_t lddy, int64_t lddx, int dtype, void* stream);

/* Widest row fk_softmax_rows_backward accepts for dtype (16384 fp32, 32768
 * bf16), or FK_ERR_INVALID_ARG for an unknown dtype. Pure host query. */
int64_t fk_softmax_backward_max_cols(int dtype);

/* Epilogue activations of fk_linear_gelu. */
typedef enum {
    FK_ACT_NONE = 0,
    FK_ACT_GELU_TANH = 1, /* the tanh-GELU of fk_gelu_tanh */
    FK_ACT_RELU = 2       /* v > 0 ? v : +0, NaN kept     */
} fk_activation;

/*
 * Linear layer with a fused activation epilogue on the matrix cores:
 * y[i][j] = act(sum_k x[i][k] w[j][k] + bias[j]), i < M, j < N, act one of
 * fk_activation (else FK_ERR_INVALID_ARG): the Linear -> GELU part of the
 * LayerNorm -> Linear -> GELU fusion example of "Lecture 6: GPU Kernels and
 * Triton", section 6.1, with the activation applied to the fp32
 * accumulators instead of a second pass over the M x N product. x: M rows of K (row stride ldx),
 * w: N rows of K (a Linear weight, row stride ldw), bias: N values or NULL,
 * y: M rows of N (row stride ldy); all DEVICE memory of dtype. fp32
 * accumulation; y rounded once to the dtype (nearest even).
 * Supported: dtype FK_BF16 or FK_F16; K < 2^36, and K, ldx and ldw
 * multiples of 8; x and w 16-byte aligned -- else FK_ERR_UNSUPPORTED. y must not overlap x, w or
 * bias (FK_ERR_OVERLAP). M == 0 or N == 0: nothing to do. K == 0 gives
 * GELU(bias).
 */
int fk_linear_gelu(const void* x, const void* w, const void* bias, void* y,
                   int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw,
                   int64_t ldy, int act, int dtype, void* stream);

/*
 * FlashAttention forward: for every batch b < B and head h < H,
 * O = softmax(Q K^T / sqrt(d) + mask) V over T positions, without forming
 * the T x T scores in HBM ("Lecture 6: GPU Kernels and Triton", sections
 * 7.3 and 8: blocks of queries against blocks of keys, online softmax with
 * a running max, sum and output accumulator, one division at the end).
 * causal = 1 keeps key j for query i when j <= i; causal = 0 keeps all.
 * q, k, v, o: DEVICE tensors [B, H, T, d] of dtype addressed by strides
 * (host array of 12 element strides: batch, head and row stride of q, then
 * of k, v, o; the d values of a row are contiguous). fp32 statistics and
 * accumulators; P is rounded to the data dtype before the P V product (as
 * the page's kernel rounds P to V's dtype); O rounded once to the dtype.
 * Supported: dtype FK_BF16 or FK_F16 (the pages benchmark fp16), d == 128,
 * 16-byte aligned bases, strides that
 * are multiples of 8, B * H * ceil(T / 128) <= 2^23 (at most one workgroup
 * per 128 queries of one head) -- else FK_ERR_UNSUPPORTED. o must not
 * overlap q, k or v (FK_ERR_OVERLAP). B, H or T == 0: nothing to do.
 */
int fk_attention_fwd(const void* q, const void* k, const void* v, void* o,
                     int64_t B, int64_t H, int64_t T, int64_t d,
                     const int64_t* strides, int causal, int dtype,
                     void* stream);

/*
 * Widest row (in columns) that fk_softmax_rows holds on chip for dtype, or
 * FK_ERR_INVALID_ARG for an unknown dtype. Pure host query.
 */
int64_t fk_softmax_onchip_max_cols(int dtype);

/*
 * Byte copy y[0 .. nbytes) = x[0 .. nbytes), through the same 128-bit
 * load/store path as the elementwise kernels: the bandwidth ceiling against
 * which the kernels' achieved bytes / time is compared ("Lecture 6: GPU
 * Kernels and Triton", section 9.3: bandwidth utilisation = bytes moved /
 * time / peak). Overlapping ranges other than x == y are FK_ERR_OVERLAP.
 */
int fk_copy(const void* x, void* y, int64_t nbytes, void* stream);

/* Static English text for an fk_status value (never NULL). */
const char* fk_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FUSEDOPS_H */
