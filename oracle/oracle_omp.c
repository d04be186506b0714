/*
 * All-cores harness around the CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY (the benchmark's CPU-baseline leg).  It runs the
 * unchanged oracle functions of oracle.c with OpenMP over independent pieces
 * of work -- tensors of a batch, row ranges of one tensor, rows of the logits
 * -- on every host core.  It adds no arithmetic of the method: the only value
 * it combines itself is a tensor's maximum magnitude from the maxima of its
 * rows, which is exact in any order, and the mean of the per-row KL losses,
 * summed in row order as the oracle does.  Results equal the single-threaded
 * calls bit for bit.
 */
#include <omp.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static size_t esize(int dtype) { return dtype == 1 ? 2 : 4; }

int orc_omp_threads(void) { return omp_get_max_threads(); }

/* B tensors of R x C elements, one orc_nvfp4_quantize call per tensor */
void orc_omp_quantize_batch(const void* x, int dtype, int64_t B, int64_t R, int64_t C,
                            uint8_t* codes, uint8_t* scales, float* tscale, uint16_t* y)
{
    const int64_t n = R * C;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b)
        orc_nvfp4_quantize((const char*)x + (size_t)(b * n) * esize(dtype), dtype, R, C, NULL, NULL,
                           codes ? codes + b * n / 2 : NULL, scales ? scales + b * n / 16 : NULL,
                           tscale ? tscale + b : NULL, y ? y + b * n : NULL);
}

/* maximum magnitude of one tensor from the maxima of its rows */
static float tensor_amax(const void* x, int dtype, int64_t R, int64_t C)
{
    float am = 0.0f;
#pragma omp parallel for reduction(max : am)
    for (int64_t r = 0; r < R; ++r) {
        const float a = orc_amax((const char*)x + (size_t)(r * C) * esize(dtype), dtype, C);
        if (a > am) am = a;
    }
    return am;
}

/* one R x C tensor (dynamic scales, or the frozen ones given), row by row */
void orc_omp_quantize_tensor(const void* x, int dtype, int64_t R, int64_t C, const uint8_t* scales_in,
                             const float* tscale_in, uint8_t* codes, uint8_t* scales, float* tscale, uint16_t* y)
{
    const float s_g = tscale_in ? *tscale_in : orc_tensor_scale(tensor_amax(x, dtype, R, C));
    if (tscale) *tscale = s_g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        orc_nvfp4_quantize_blocks((const char*)x + (size_t)(r * C) * esize(dtype), dtype, C / 16, s_g,
                                  scales_in ? scales_in + r * C / 16 : NULL, codes ? codes + r * C / 2 : NULL,
                                  scales ? scales + r * C / 16 : NULL, y ? y + r * C : NULL);
}

/* MSE calibration of one R x C tensor, row by row */
void orc_omp_mse_calibrate(const void* x, int dtype, int64_t R, int64_t C, int n_cand, float k_min, float k_max,
                           uint8_t* scales, float* tscale)
{
    const float s_g = orc_tensor_scale(tensor_amax(x, dtype, R, C));
    if (tscale) *tscale = s_g;
#pragma omp parallel
    {
        float* row = (float*)malloc(sizeof(float) * (size_t)C);
#pragma omp for schedule(static)
        for (int64_t r = 0; r < R; ++r) {
            if (dtype == 1) {
                const uint16_t* h = (const uint16_t*)x + r * C;
                for (int64_t c = 0; c < C; ++c) row[c] = orc_f32_from_bf16(h[c]);
            } else {
                memcpy(row, (const float*)x + r * C, sizeof(float) * (size_t)C);
            }
            orc_mse_calibrate_blocks(row, C / 16, s_g, n_cand, k_min, k_max, scales + r * C / 16, NULL, NULL, NULL);
        }
        free(row);
    }
}

/* KL loss and gradient of `rows` rows, one orc_kl_fwd_bwd call per row;
 * row_kl is required; returns the mean over rows */
double orc_omp_kl_fwd_bwd(const void* teacher, const void* student, int dtype, int64_t rows, int64_t V, double T,
                          double grad_scale, double* row_kl, double* grad)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        const size_t off = (size_t)(r * V) * esize(dtype);
        orc_kl_fwd_bwd((const char*)teacher + off, (const char*)student + off, dtype, 1, V, T, grad_scale,
                       row_kl + r, grad ? grad + r * V : NULL);
    }
    double total = 0.0;
    for (int64_t r = 0; r < rows; ++r) total += row_kl[r];
    return rows > 0 ? total / (double)rows : 0.0;
}

/* the binary32 timing variant, one row per call */
float orc_omp_kl_fwd_bwd_f32(const void* teacher, const void* student, int dtype, int64_t rows, int64_t V, float T,
                             float grad_scale, float* row_kl, float* grad)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        const size_t off = (size_t)(r * V) * esize(dtype);
        orc_kl_fwd_bwd_f32((const char*)teacher + off, (const char*)student + off, dtype, 1, V, T, grad_scale,
                           row_kl + r, grad ? grad + r * V : NULL);
    }
    double total = 0.0;
    for (int64_t r = 0; r < rows; ++r) total += row_kl[r];
    return rows > 0 ? (float)(total / (double)rows) : 0.0f;
}
