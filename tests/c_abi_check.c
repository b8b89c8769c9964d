/* c_abi_check.c -- the C ABI used from plain C99: include/fusedops.h must
 * compile as C and libfusedops.so must link and answer from C. Only calls
 * that return before any HIP call are made (queries and argument errors),
 * so this runs without a GPU. Prints "ok" and exits 0 when every check
 * holds; otherwise prints the failed check and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fusedops.h"

static int failures = 0;

#define CHECK(cond)                                            \
    do {                                                       \
        if (!(cond)) {                                         \
            printf("failed: %s (line %d)\n", #cond, __LINE__); \
            ++failures;                                        \
        }                                                      \
    } while (0)

int main(void) {
    /* plausible, 16-byte aligned fake device addresses 1 GiB apart: never
       dereferenced, since every call below is refused by the host-side
       checks (or has no work) before anything is enqueued */
    char* a = (char*)(uintptr_t)0x7F0000000000ull;
    char* b = (char*)(uintptr_t)0x7F0040000000ull;
    char* c = (char*)(uintptr_t)0x7F0080000000ull;
    char* o = (char*)(uintptr_t)0x7F00C0000000ull;
    fk_op ops[FK_MAX_OPS + 1];
    int64_t strides[12];
    int i;
    for (i = 0; i < FK_MAX_OPS + 1; ++i) {
        ops[i].kind = FK_OP_ADD_SCALAR;
        ops[i].scalar = 1.0f;
    }
    for (i = 0; i < 4; ++i) {  /* per operand: batch, head, row strides (elements) */
        strides[3 * i] = 8 * 128;
        strides[3 * i + 1] = 8 * 128;
        strides[3 * i + 2] = 128;
    }

    CHECK(strcmp(fk_status_string(FK_OK), fk_status_string(FK_ERR_HIP)) != 0);
    CHECK(fk_status_string(FK_ERR_OVERLAP) != NULL);

    /* capacity queries */
    CHECK(fk_softmax_onchip_max_cols(FK_F32) == 32768);
    CHECK(fk_softmax_onchip_max_cols(FK_BF16) == 65536);
    CHECK(fk_layernorm_max_cols(FK_F32) == 32768);
    CHECK(fk_softmax_backward_max_cols(FK_BF16) == 32768);
    CHECK(fk_softmax_workspace_bytes(16, 1000, FK_F32) == 0);      /* on chip: none */
    CHECK(fk_softmax_workspace_bytes(1024, 131072, FK_F32) == 1024 * 16 * 16); /* split rows */
    CHECK(fk_softmax_rows_path(a, b, 1024, 131072, 131072, 131072, FK_F32, 0) == FK_PATH_ONLINE);
    CHECK(fk_softmax_rows_path(a, b, 1024, 131072, 131072, 131072, FK_F32, 1 << 18) ==
          FK_PATH_SPLIT);
    CHECK(fk_softmax_rows_path(a, a, 1024, 131072, 131072, 131072, FK_F32, 1 << 18) ==
          FK_PATH_ONLINE);
    CHECK(fk_softmax_rows_path(a, b, 16, 1000, 1000, 1000, FK_F32, 0) == FK_PATH_ONCHIP);

    /* empty work: FK_OK, nothing launched, NULL pointers allowed */
    CHECK(fk_gelu_tanh(NULL, NULL, 0, FK_F32, NULL) == FK_OK);
    CHECK(fk_softmax_rows(NULL, NULL, 0, 10, 10, 10, FK_BF16, NULL) == FK_OK);

    /* argument errors */
    CHECK(fk_gelu_tanh(a, b, -1, FK_F32, NULL) == FK_ERR_INVALID_ARG);
    CHECK(fk_gelu_tanh(NULL, b, 4, FK_F32, NULL) == FK_ERR_INVALID_ARG);
    CHECK(fk_gelu_tanh(a, b, 4, 7, NULL) == FK_ERR_INVALID_ARG);
    CHECK(fk_gelu_tanh(a, b, 4, FK_F16, NULL) == FK_ERR_UNSUPPORTED);
    CHECK(fk_gelu_tanh(a, a + 4, 4, FK_F32, NULL) == FK_ERR_OVERLAP);
    CHECK(fk_elementwise_chain(a, b, 4, FK_F32, ops, 0, NULL) == FK_ERR_INVALID_ARG);
    CHECK(fk_elementwise_chain(a, b, 4, FK_F32, ops, FK_MAX_OPS + 1, NULL) == FK_ERR_INVALID_ARG);
    CHECK(fk_softmax_rows(a, b, 2, 8, 4, 8, FK_F32, NULL) == FK_ERR_INVALID_ARG);   /* ldx < cols */
    CHECK(fk_softmax_rows_online(a, b, -1, 8, 8, 8, FK_F32, NULL) == FK_ERR_INVALID_ARG);
    CHECK(fk_layernorm_rows(a, b, 2, 32769, 32769, 32769, NULL, NULL, 1e-5f, 0, FK_F32, NULL) ==
          FK_ERR_UNSUPPORTED);
    CHECK(fk_gelu_tanh_backward(a, b, c, 4, FK_F16, NULL) == FK_ERR_UNSUPPORTED);
    CHECK(fk_softmax_rows_backward(a, b, c, 2, 16385, 16385, 16385, 16385, FK_F32, NULL) ==
          FK_ERR_UNSUPPORTED);
    CHECK(fk_linear_gelu(a, b, NULL, c, 4, 10, 16, 16, 16, 10, 1, FK_F32, NULL) ==
          FK_ERR_UNSUPPORTED);
    CHECK(fk_attention_fwd(a, b, c, o, 1, 1, 8, 64, strides, 1, FK_BF16, NULL) ==
          FK_ERR_UNSUPPORTED);                                                   /* d != 128 */
    strides[2] = 100;                                                /* q rows shorter than d */
    CHECK(fk_attention_fwd(a, b, c, o, 1, 1, 8, 128, strides, 1, FK_BF16, NULL) ==
          FK_ERR_INVALID_ARG);
    CHECK(fk_copy(a, b, -1, NULL) == FK_ERR_INVALID_ARG);

    if (failures) return 1;
    printf("ok\n");
    return 0;
}
