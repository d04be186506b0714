/*
 * A plain C99 client of libqad that drives the host-side validation of every
 * entry point (each call fails a check before any device work, so no GPU is
 * needed), for builds of the client -- and of the library's host code --
 * under AddressSanitizer and UndefinedBehaviorSanitizer.  Prints "ok" when
 * every status matched.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "libqad.h"

static int failures = 0;

static void check(int line, qad_status_t got, qad_status_t want)
{
    if (got != want) {
        printf("line %d: got %s, want %s\n", line, qad_status_string(got), qad_status_string(want));
        ++failures;
    }
}
#define CHECK(call, want) check(__LINE__, (call), (want))

int main(void)
{
    /* fake, far-apart, 256-byte aligned addresses: never dereferenced, since
     * every call below fails validation before any device work */
    char* P = (char*)(uintptr_t)0x100000000ull;
    const size_t Q = (size_t)1 << 24;
    char* ODD = P + 2;
    const qad_dtype_t BAD = (qad_dtype_t)7;

    if (qad_abi_version() != 2) ++failures;
    for (int s = 0; s <= 8; ++s) if (!qad_status_string((qad_status_t)s)) ++failures;
    for (int op = 0; op <= 7; ++op) (void)qad_workspace_bytes((qad_op_t)op, 3, 17, 4096);
    if (qad_workspace_bytes(QAD_OP_QUANTIZE, -1, 4, 16) != 0) ++failures;
    const int64_t prev = qad_set_wait_limit_us(-1);
    (void)qad_set_wait_limit_us((int64_t)1 << 50);
    (void)qad_set_wait_limit_us(prev);

    CHECK(nvfp4_amax(P, BAD, 1, 4, 16, (float*)(P + Q), P + 2 * Q, 1 << 16, NULL), QAD_ERR_DTYPE);
    CHECK(nvfp4_amax(P, QAD_BF16, 1, 4, 12, (float*)(P + Q), P + 2 * Q, 1 << 16, NULL), QAD_ERR_SHAPE);
    CHECK(nvfp4_amax(P, QAD_BF16, 1, 4, 16, NULL, P + 2 * Q, 1 << 16, NULL), QAD_ERR_INVALID_ARG);
    CHECK(nvfp4_amax(ODD, QAD_BF16, 1, 4, 16, (float*)(P + Q), P + 2 * Q, 1 << 16, NULL), QAD_ERR_ALIGNMENT);
    CHECK(nvfp4_amax(P, QAD_BF16, 1, 4, 16, (float*)(P + Q), NULL, 0, NULL), QAD_ERR_WORKSPACE);

    CHECK(nvfp4_quantize(P, BAD, 1, 4, 32, NULL, NULL, (uint8_t*)(P + Q), NULL, NULL, NULL, P + 2 * Q, 1 << 16, NULL),
          QAD_ERR_DTYPE);
    CHECK(nvfp4_quantize(P, QAD_BF16, 1, 4, 24, NULL, NULL, (uint8_t*)(P + Q), NULL, NULL, NULL, P + 2 * Q, 1 << 16,
                         NULL), QAD_ERR_SHAPE);
    CHECK(nvfp4_quantize(P, QAD_BF16, 1, 4, 32, NULL, NULL, NULL, NULL, NULL, NULL, P + 2 * Q, 1 << 16, NULL),
          QAD_ERR_INVALID_ARG);
    CHECK(nvfp4_quantize(P, QAD_BF16, 1, 4, 32, NULL, NULL, (uint8_t*)(P + Q), NULL, NULL, NULL, NULL, 0, NULL),
          QAD_ERR_WORKSPACE);
    CHECK(nvfp4_quantize(P, QAD_BF16, 1, 4, 32, NULL, NULL, (uint8_t*)P, NULL, NULL, NULL, P + 2 * Q, 1 << 16,
                         NULL), QAD_ERR_INVALID_ARG);   /* codes over x */
    CHECK(nvfp4_quantize_noalloc(P, BAD, 1, 4, 32, NULL, NULL, (uint8_t*)(P + Q), NULL, NULL, NULL, NULL),
          QAD_ERR_DTYPE);
    CHECK(nvfp4_quantize_noalloc(P, QAD_BF16, 65536, 1, 16, NULL, NULL, NULL, NULL, NULL, P + Q, NULL),
          QAD_ERR_WORKSPACE);   /* records beyond the fixed scratch */
    CHECK(nvfp4_qdq_fwd(P, QAD_BF16, 1, 4, 24, NULL, NULL, P + Q, P + 2 * Q, 1 << 16, NULL), QAD_ERR_SHAPE);
    CHECK(nvfp4_qdq_bwd(NULL, P + Q, QAD_BF16, 100, NULL), QAD_ERR_INVALID_ARG);
    CHECK(nvfp4_qdq_bwd(P, P + 64, QAD_BF16, 100, NULL), QAD_ERR_INVALID_ARG);
    CHECK(nvfp4_qdq_bwd(P, P + Q, BAD, 100, NULL), QAD_ERR_DTYPE);
    CHECK(nvfp4_qdq_bwd_clipped(P, QAD_BF16, P + Q, QAD_BF16, 2, 4, 24, (uint8_t*)(P + 2 * Q), (float*)(P + 3 * Q),
                                P + 4 * Q, NULL), QAD_ERR_SHAPE);
    CHECK(nvfp4_qdq_bwd_clipped(P, QAD_BF16, P + Q, QAD_BF16, 2, 4, 32, (uint8_t*)(P + 2 * Q), (float*)(P + 3 * Q),
                                P + Q, NULL), QAD_ERR_INVALID_ARG);   /* grad_x over x */
    CHECK(nvfp4_frozen_sgd_step(P, QAD_BF16, P + Q, QAD_BF16, 2, 4, 32, (uint8_t*)(P + 2 * Q), (float*)(P + 3 * Q),
                                0.5f, 1.0f / 0.0f, P + 4 * Q, NULL), QAD_ERR_INVALID_ARG);
    CHECK(nvfp4_frozen_sgd_step(P, BAD, P + Q, QAD_BF16, 2, 4, 32, (uint8_t*)(P + 2 * Q), (float*)(P + 3 * Q),
                                0.5f, 1.0f, P + 4 * Q, NULL), QAD_ERR_DTYPE);
    CHECK(nvfp4_frozen_sgd_step(P, QAD_BF16, P + Q, QAD_BF16, 2, 4, 32, (uint8_t*)(P + 2 * Q), (float*)(P + 3 * Q),
                                0.5f, 1.0f, P + Q, NULL), QAD_ERR_INVALID_ARG);   /* w_out over grad */
    CHECK(nvfp4_mse_calibrate(P, QAD_BF16, 1, 4, 32, 0, 0.5f, 1.0f, (uint8_t*)(P + Q), (float*)(P + 2 * Q),
                              P + 3 * Q, 1 << 16, NULL), QAD_ERR_INVALID_ARG);
    CHECK(nvfp4_mse_calibrate(P, QAD_BF16, 1, 4, 32, 64, 0.1f, 1.0f, (uint8_t*)(P + Q), (float*)(P + 2 * Q),
                              P + 3 * Q, 1 << 16, NULL), QAD_ERR_INVALID_ARG);   /* grid too coarse */
    CHECK(fp8_quantize(P, QAD_BF16, 1, 4, 12, NULL, (uint8_t*)(P + Q), NULL, NULL, P + 2 * Q, 1 << 16, NULL),
          QAD_ERR_SHAPE);
    CHECK(qad_w4a4_linear_fwd(P, P + Q, BAD, 8, 8, 32, NULL, NULL, P + 2 * Q, P + 3 * Q, P + 4 * Q, P + 5 * Q, 1 << 20,
                              NULL), QAD_ERR_DTYPE);
    CHECK(qad_w4a4_linear_fwd(P, P + Q, QAD_BF16, 8, 8, 24, NULL, NULL, P + 2 * Q, P + 3 * Q, P + 4 * Q, P + 5 * Q,
                              1 << 20, NULL), QAD_ERR_SHAPE);
    CHECK(qad_w4a4_linear_bwd(P, P + Q, P + 2 * Q, 8, 8, 32, NULL, NULL, P + 3 * Q, 1 << 20, NULL),
          QAD_ERR_INVALID_ARG);
    CHECK(qad_kl_fwd_bwd(P, P + Q, BAD, 4, 64, 1.0f, 0.25f, (float*)(P + 2 * Q), NULL, NULL, QAD_BF16, P + 3 * Q,
                         1 << 20, NULL), QAD_ERR_DTYPE);
    CHECK(qad_kl_fwd_bwd(P, P + Q, QAD_BF16, 4, 64, 0.0f, 0.25f, (float*)(P + 2 * Q), NULL, NULL, QAD_BF16,
                         P + 3 * Q, 1 << 20, NULL), QAD_ERR_INVALID_ARG);   /* T = 0 */
    CHECK(qad_kl_fwd_bwd(P, P + Q, QAD_BF16, 4, 63, 1.0f, 0.25f, (float*)(P + 2 * Q), NULL, NULL, QAD_BF16,
                         P + 3 * Q, 1 << 20, NULL), QAD_ERR_SHAPE);
    CHECK(qad_kl_topk_fwd_bwd(P, P + Q, QAD_BF16, 4, 64, 0, 1.0f, 0.25f, (float*)(P + 2 * Q), NULL, NULL, QAD_BF16,
                              P + 3 * Q, 1 << 20, NULL), QAD_ERR_INVALID_ARG);   /* k = 0 */
    CHECK(qad_kl_topp_fwd_bwd(P, P + Q, QAD_BF16, 4, 64, 0.0f, 1.0f, 0.25f, (float*)(P + 2 * Q), NULL, NULL,
                              QAD_BF16, NULL, P + 3 * Q, 1 << 20, NULL), QAD_ERR_INVALID_ARG);   /* top_p = 0 */
    CHECK(qad_check_finite(NULL, 4, NULL), QAD_ERR_INVALID_ARG);
    if (failures) return 1;
    printf("ok\n");
    return 0;
}
