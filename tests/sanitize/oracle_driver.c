/*
 * Drives every oracle entry point (and the all-cores harness) on small
 * inputs, edge cases included, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Prints "ok" when every call returned; any
 * out-of-bounds access, leak or undefined operation aborts the program.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint16_t bf16_of(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int main(void)
{
    enum { R = 5, C = 48, N = R * C, V = 40 };
    float xf[N];
    uint16_t xb[N], gb[N];
    srand(7);
    for (int i = 0; i < N; ++i) {
        xf[i] = ((float)rand() / RAND_MAX - 0.5f) * (i % 17 == 0 ? 300.0f : 3.0f);
        xb[i] = bf16_of(xf[i]);
        gb[i] = bf16_of(((float)rand() / RAND_MAX - 0.5f));
    }
    xf[3] = 0.0f;
    xf[4] = -0.0f;
    xf[5] = 1e-40f;   /* subnormal */

    /* codecs */
    for (int c = 0; c < 256; ++c) (void)orc_e4m3_decode((uint8_t)c);
    for (int c = 0; c < 16; ++c) (void)orc_e2m1_decode((uint8_t)c);
    const float probes[] = {0.0f, -0.0f, 0.25f, 0.75f, 5.0f, 6.5f, 1e30f, -448.0f, 464.0f, 1e-45f};
    for (size_t i = 0; i < sizeof probes / sizeof probes[0]; ++i) {
        (void)orc_e2m1_encode(probes[i]);
        (void)orc_e4m3_encode(fabsf(probes[i]));
        (void)orc_f32_from_bf16(orc_bf16_from_f32(probes[i]));
    }

    uint8_t codes[N / 2], scales[N / 16], codes8[N];
    uint16_t y[N], out_b[N];
    float ts, out_f[N];
    int64_t n_clip = 0;

    /* NVFP4: dynamic, frozen, blocks; fp32 and bf16 inputs */
    orc_nvfp4_quantize(xf, 0, R, C, NULL, NULL, codes, scales, &ts, y);
    orc_nvfp4_quantize(xb, 1, R, C, NULL, NULL, codes, scales, &ts, y);
    orc_nvfp4_quantize(xb, 1, R, C, scales, &ts, codes, NULL, NULL, y);
    orc_nvfp4_quantize_blocks(xf, 0, N / 16, ts, NULL, codes, scales, y);
    orc_nvfp4_quantize(xf, 0, 0, C, NULL, NULL, codes, scales, &ts, y);   /* empty */
    (void)orc_amax(xb, 1, N);
    (void)orc_tensor_scale(0.0f);

    /* FP8 */
    orc_fp8_quantize(xf, 0, N, NULL, codes8, &ts, y);
    orc_fp8_quantize(xb, 1, N, &ts, codes8, NULL, y);

    /* MSE: the usual grid, a one-candidate grid and one beyond 4096 */
    float kg[64];
    orc_mse_kgrid(64, 0.5f, 1.0f, kg);
    orc_mse_calibrate(xb, 1, R, C, 64, 0.5f, 1.0f, scales, &ts);
    orc_mse_calibrate(xf, 0, R, C, 1, 1.0f, 1.0f, scales, &ts);
    orc_mse_calibrate(xf, 0, 1, 16, 5000, 0.5f, 1.0f, scales, &ts);
    float err[N / 16];
    uint8_t cc[2 * 70];
    float ce[2 * 70];
    orc_mse_calibrate_blocks(xf, 2, ts, 70, 0.5f, 1.0f, scales, err, cc, ce);

    /* clipped STE and the frozen-scale step */
    orc_nvfp4_qdq_bwd_clipped(gb, 1, xb, 1, N / 16, scales, ts, out_b, &n_clip);
    orc_nvfp4_qdq_bwd_clipped(xf, 0, xf, 0, N / 16, scales, ts, out_f, &n_clip);
    orc_nvfp4_frozen_sgd_step(xb, 1, gb, 1, N / 16, scales, ts, 0.5f, 0.25f, out_b, &n_clip);
    orc_nvfp4_frozen_sgd_step(xf, 0, gb, 1, N / 16, scales, ts, 0.5f, 0.25f, out_f, &n_clip);

    /* KL, top-k, top-p, the binary32 variant */
    uint16_t tb[3 * V], sb[3 * V];
    for (int i = 0; i < 3 * V; ++i) {
        tb[i] = bf16_of(((float)rand() / RAND_MAX - 0.5f) * 6.0f);
        sb[i] = bf16_of(((float)rand() / RAND_MAX - 0.5f) * 6.0f);
    }
    double row[3], grad[3 * V], tau[3], mass[6];   /* mass: two per row */
    int64_t cnt[3];
    float rowf[3], gradf[3 * V];
    (void)orc_kl_fwd_bwd(tb, sb, 1, 3, V, 1.0, 1.0 / 3, row, grad);
    (void)orc_kl_fwd_bwd(tb, tb, 1, 3, V, 0.5, 1.0 / 3, row, NULL);
    (void)orc_kl_topk_fwd_bwd(tb, sb, 1, 3, V, 7, 1.0, 1.0 / 3, row, grad, cnt);
    (void)orc_kl_topk_fwd_bwd(tb, sb, 1, 3, V, 1000, 2.0, 1.0 / 3, row, grad, cnt);
    (void)orc_kl_topp_fwd_bwd(tb, sb, 1, 3, V, 0.9, 1.0, 1.0 / 3, row, grad, cnt, tau, mass);
    (void)orc_kl_topp_fwd_bwd(tb, sb, 1, 3, V, 1.0, 1.0, 1.0 / 3, row, grad, cnt, tau, mass);
    (void)orc_kl_fwd_bwd_f32(tb, sb, 1, 3, V, 1.0f, 1.0f / 3, rowf, gradf);

    /* the all-cores harness */
    float tsb[R];
    uint8_t codes_b[N / 2], scales_b[N / 16];
    uint16_t yb[N];
    (void)orc_omp_threads();
    orc_omp_quantize_batch(xb, 1, R, 1, C, codes_b, scales_b, tsb, yb);
    orc_omp_quantize_tensor(xf, 0, R, C, NULL, NULL, codes, scales, &ts, y);
    orc_omp_quantize_tensor(xb, 1, R, C, scales, &ts, codes, NULL, NULL, y);
    orc_omp_mse_calibrate(xb, 1, R, C, 64, 0.5f, 1.0f, scales, &ts);
    (void)orc_omp_kl_fwd_bwd(tb, sb, 1, 3, V, 1.0, 1.0 / 3, row, grad);
    (void)orc_omp_kl_fwd_bwd_f32(tb, sb, 1, 3, V, 1.0f, 1.0f / 3, rowf, gradf);
    printf("ok\n");
    return 0;
}
