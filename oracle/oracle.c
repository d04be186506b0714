/*
 * CPU oracle for the QAD hot path (NVFP4 simulated quantization + KL loss).
 * TEST INFRASTRUCTURE ONLY -- see oracle.h for the page legend, the
 * precision rules and who may use this file.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared (no fast-math).
 * On x86-64 every `float` operation below is one IEEE binary32 operation
 * rounded to nearest-even; nothing is fused or reassociated.
 */
#include "oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float    u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ------------------------------------------------------------------------
 * E2M1 ("4-bit floating point", [Nano] section "NVFP4-Format und warum es
 * wichtig ist?").  The pages name the format but not its grid; the reading
 * taken is the standard E2M1 layout: 1 sign bit, 2 exponent bits (bias 1),
 * 1 mantissa bit, exponent 0 subnormal -> magnitudes
 *     idx : 0    1    2    3    4    5    6    7
 *     val : 0   0.5   1   1.5   2    3    4    6
 * Rounding: nearest grid value, ties to the even index, magnitudes beyond 6
 * saturate to 6.  Written as the midpoints between neighbouring grid values:
 * at a midpoint the even index wins, so the comparison is "<=" when the lower
 * neighbour is even and "<" when it is odd.
 * ---------------------------------------------------------------------- */
static const float E2M1_VAL[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

static unsigned e2m1_index(float a) /* a = |r|, finite */
{
    if (a <= 0.25f) return 0; /* midpoint 0|0.5,   lower idx 0 even */
    if (a <  0.75f) return 1; /* midpoint 0.5|1,   lower idx 1 odd  */
    if (a <= 1.25f) return 2; /* midpoint 1|1.5,   lower idx 2 even */
    if (a <  1.75f) return 3; /* midpoint 1.5|2,   lower idx 3 odd  */
    if (a <= 2.5f)  return 4; /* midpoint 2|3,     lower idx 4 even */
    if (a <  3.5f)  return 5; /* midpoint 3|4,     lower idx 5 odd  */
    if (a <= 5.0f)  return 6; /* midpoint 4|6,     lower idx 6 even */
    return 7;                 /* (5, inf): 6, saturating            */
}

uint8_t orc_e2m1_encode(float r)
{
    unsigned sign = f2u(r) >> 31;   /* signbit: -0 gives a negative code */
    float a = fabsf(r);
    if (isnan(a)) a = INFINITY;     /* not expected; saturate deterministically */
    return (uint8_t)((sign << 3) | e2m1_index(a));
}

float orc_e2m1_decode(uint8_t code)
{
    float v = E2M1_VAL[code & 7];
    return (code & 8) ? -v : v;
}

void orc_e2m1_encode_array(const float* r, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_encode(r[i]);
}

/* ------------------------------------------------------------------------
 * E4M3 block scale ("E4M3-FP8" per block, [Nano] section "NVFP4-Format und
 * warum es wichtig ist?").  Reading: the OCP "E4M3FN" encoding -- bias 7,
 * largest finite 448 (code 0x7E), no infinities, 0x7F is NaN (never
 * produced), subnormals m * 2^-9.  Encoding rounds to nearest-even and
 * saturates at 448.  Scales are non-negative, so only the positive half is
 * encoded.
 * ---------------------------------------------------------------------- */
float orc_e4m3_decode(uint8_t code)
{
    unsigned e = (code >> 3) & 15, m = code & 7;
    float v;
    if ((code & 0x7F) == 0x7F) return NAN;
    if (e == 0) v = ldexpf((float)m, -9);                 /* m * 2^-9          */
    else        v = ldexpf(1.0f + (float)m / 8.0f, (int)e - 7);
    return (code & 0x80) ? -v : v;
}

uint8_t orc_e4m3_encode(float v)
{
    /* v >= 0 and finite */
    if (!(v > 0.0f)) return 0;                            /* 0 (and -0)        */
    if (v > 448.0f) return 0x7E;                          /* saturate (also +inf) */
    if (v >= 0.015625f) {                                 /* normal: v >= 2^-6 */
        int E;
        float f = frexpf(v, &E);                          /* v = f * 2^E, f in [0.5,1) */
        E -= 1;                                           /* v = (2f) * 2^E, 2f in [1,2) */
        float frac = ldexpf(f, 1) - 1.0f;                 /* exact, in [0,1)   */
        float m = nearbyintf(frac * 8.0f);                /* RNE, exact scaling */
        if (m == 8.0f) { m = 0.0f; E += 1; }              /* mantissa carry    */
        int biased = E + 7;
        if (biased > 15) return 0x7E;                     /* beyond the format: saturate */
        unsigned code = ((unsigned)biased << 3) | (unsigned)m;
        if (code > 0x7E) code = 0x7E;                     /* 480 would be NaN: saturate */
        return (uint8_t)code;
    } else {                                              /* subnormal range   */
        float m = nearbyintf(ldexpf(v, 9));               /* v*2^9 exact, RNE  */
        return (uint8_t)m;                                /* m == 8 is code 0x08 = 2^-6 */
    }
}

void orc_e4m3_encode_array(const float* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

/* ------------------------------------------------------------------------
 * bfloat16: top 16 bits of binary32, rounded to nearest-even.
 * ---------------------------------------------------------------------- */
uint16_t orc_bf16_from_f32(float f)
{
    uint32_t u = f2u(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x40);    /* quiet NaN         */
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

float orc_f32_from_bf16(uint16_t h) { return u2f((uint32_t)h << 16); }

void orc_bf16_from_f32_array(const float* f, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f32(f[i]);
}

/* element i of an input tensor as binary32 (bf16 -> fp32 is exact) */
static float load_x(const void* x, int dtype, int64_t i)
{
    if (dtype == 1) return orc_f32_from_bf16(((const uint16_t*)x)[i]);
    return ((const float*)x)[i];
}

/* ------------------------------------------------------------------------
 * Tensor amax: the largest magnitude over the whole tensor.  Max calibration
 * is what the dynamic-scale variant starts from ([Lightning] section
 * "量化尺度处理策略", dynamic-scale QAD recomputes it every step).
 * ---------------------------------------------------------------------- */
float orc_amax(const void* x, int dtype, int64_t n)
{
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(load_x(x, dtype, i));
        if (a > m || isnan(a)) m = a;
    }
    return m;
}

/* Two-level scaling ([Nano]: FP32 scale per tensor, E4M3 scale per block).
 * Reading: the tensor scale maps the tensor amax onto the product of the
 * largest E2M1 value (6) and the largest E4M3 value (448), so that the block
 * holding the tensor amax gets the largest block scale.  An all-zero tensor
 * gets tensor scale 1. */
float orc_tensor_scale(float amax)
{
    return amax > 0.0f ? amax / 2688.0f : 1.0f;
}

/* E4M3 block scale of a block with amax amax_b under tensor scale s_g:
 * the block amax is mapped onto 6 (the top of the E2M1 grid), expressed in
 * units of the tensor scale, then rounded to E4M3. */
static uint8_t block_scale_code(float amax_b, float s_g)
{
    float per_block = amax_b / 6.0f;
    float raw = per_block / s_g;
    return orc_e4m3_encode(raw);
}

/* Quantize one 16-element block with effective scale s_eff = dec(s_b) * s_g.
 * code = E2M1(x / s_eff) with the quotient correctly rounded to binary32;
 * a zero effective scale gives signed-zero codes (no division).  The
 * dequantized value is the binary32 product dec(code) * s_eff rounded once
 * more to bf16. */
static void quantize_block(const float* xb, float s_eff, uint8_t* code16, uint16_t* y16)
{
    for (int j = 0; j < 16; ++j) {
        uint8_t c;
        if (s_eff == 0.0f) {
            c = (uint8_t)((f2u(xb[j]) >> 31) << 3);
        } else {
            float r = xb[j] / s_eff;
            c = orc_e2m1_encode(r);
        }
        code16[j] = c;
        float deq = orc_e2m1_decode(c) * s_eff;   /* +-0 stays +-0 */
        y16[j] = orc_bf16_from_f32(deq);
    }
}

/* Quantize nb consecutive blocks under tensor scale s_g; block scales are
 * computed from each block (dynamic) unless scales_in supplies them (frozen). */
static void quantize_blocks(const void* x, int dtype, int64_t nb, float s_g,
                            const uint8_t* scales_in, uint8_t* codes, uint8_t* scales,
                            uint16_t* y)
{
    float xb[16];
    uint8_t c16[16];
    uint16_t y16[16];
    for (int64_t b = 0; b < nb; ++b) {
        float amax_b = 0.0f;
        for (int j = 0; j < 16; ++j) {
            xb[j] = load_x(x, dtype, b * 16 + j);
            float a = fabsf(xb[j]);
            if (a > amax_b) amax_b = a;
        }
        uint8_t sb = scales_in ? scales_in[b] : block_scale_code(amax_b, s_g);
        float s_eff = orc_e4m3_decode(sb) * s_g;
        quantize_block(xb, s_eff, c16, y16);
        if (scales) scales[b] = sb;
        if (codes)
            for (int j = 0; j < 16; j += 2)
                codes[b * 8 + j / 2] = (uint8_t)((c16[j] & 15) | ((c16[j + 1] & 15) << 4));
        if (y) memcpy(y + b * 16, y16, sizeof y16);
    }
}

void orc_nvfp4_quantize(const void* x, int dtype, int64_t R, int64_t C,
                        const uint8_t* scales_in, const float* tscale_in,
                        uint8_t* codes, uint8_t* scales, float* tscale,
                        uint16_t* y)
{
    const int64_t n = R * C;
    float s_g;
    if (scales_in) {
        s_g = *tscale_in;                              /* frozen: stored tensor scale */
    } else {
        s_g = orc_tensor_scale(orc_amax(x, dtype, n)); /* dynamic: recomputed         */
    }
    if (tscale) *tscale = s_g;
    quantize_blocks(x, dtype, n / 16, s_g, scales_in, codes, scales, y);
}

void orc_nvfp4_quantize_blocks(const void* x, int dtype, int64_t nblocks, float s_g,
                               const uint8_t* scales_in, uint8_t* codes, uint8_t* scales,
                               uint16_t* y)
{
    quantize_blocks(x, dtype, nblocks, s_g, scales_in, codes, scales, y);
}

/* ------------------------------------------------------------------------
 * Clipped straight-through backward.  [Lightning] section "量化尺度处理策略":
 * with frozen scales only the weights train, the scales stay fixed.  The
 * pages print no clipping rule; the reading taken is the usual one for a
 * saturating quantizer: the gradient passes where the element lies inside the
 * range its block can represent, |x| <= 6 * s_eff, and is +0 where the
 * quantizer saturates.  s_eff = fl(dec(s_b) * s_g) is the forward's binary32
 * effective scale; the comparison is exact (6 * s_eff needs at most 26
 * significant bits, so the binary64 product is exact).  The scales are the
 * ones the forward used (frozen, or the dynamic ones it reported).
 * ---------------------------------------------------------------------- */
void orc_nvfp4_qdq_bwd_clipped(const void* grad_y, int gdtype, const void* x, int xdtype,
                               int64_t nblocks, const uint8_t* scales, float s_g,
                               void* grad_x, int64_t* n_clipped)
{
    int64_t clipped = 0;
    for (int64_t b = 0; b < nblocks; ++b) {
        const float s_eff = orc_e4m3_decode(scales[b]) * s_g;
        const double lim = 6.0 * (double)s_eff;
        for (int j = 0; j < 16; ++j) {
            const int64_t i = b * 16 + j;
            const int pass = fabs((double)load_x(x, xdtype, i)) <= lim;
            clipped += !pass;
            if (gdtype == 1)
                ((uint16_t*)grad_x)[i] = pass ? ((const uint16_t*)grad_y)[i] : 0;
            else
                ((float*)grad_x)[i] = pass ? ((const float*)grad_y)[i] : 0.0f;
        }
    }
    if (n_clipped) *n_clipped = clipped;
}

/* ------------------------------------------------------------------------
 * Frozen-scale weight step.  [Lightning] section "量化尺度处理策略": with
 * frozen (MSE-calibrated) scales the scales stay fixed and only the weights
 * are updated; section "训练配置": a constant learning rate and gradient
 * clipping at norm 1.0.  The pages name no optimizer; the reading taken is
 * plain SGD whose step is the learning rate times the clipping coefficient
 * the caller derived from the global gradient norm (min(1, max_norm/norm)),
 * applied to the gradient that reaches the weight through the quantizer, i.e.
 * the clipped straight-through one above:
 *   a  = fl32(lr * clip_coef)
 *   w' = w                              where |w| > 6 * s_eff (saturated:
 *                                       no gradient reaches the weight)
 *   w' = round_w(fma32(-a, g, w))       elsewhere
 * fma32 is one binary32 rounding (to nearest even); round_w is the identity
 * for binary32 weights and a second rounding to bf16 (nearest even) for bf16
 * weights.  The weight is the forward's input (it is what the quantizer
 * coded), so the test |w| <= 6 * s_eff is exact as in the clipped backward.
 * Optional n_clipped: number of weights left unchanged by the clip.
 * ---------------------------------------------------------------------- */
void orc_nvfp4_frozen_sgd_step(const void* w, int wdtype, const void* grad, int gdtype, int64_t nblocks,
                               const uint8_t* scales, float s_g, float lr, float clip_coef, void* w_out,
                               int64_t* n_clipped)
{
    const float a = lr * clip_coef;   /* binary32 product (built with -ffp-contract=off) */
    int64_t clipped = 0;
    for (int64_t b = 0; b < nblocks; ++b) {
        const float s_eff = orc_e4m3_decode(scales[b]) * s_g;
        const double lim = 6.0 * (double)s_eff;
        for (int j = 0; j < 16; ++j) {
            const int64_t i = b * 16 + j;
            const float wv = load_x(w, wdtype, i);
            if (!(fabs((double)wv) <= lim)) {
                ++clipped;
                if (wdtype == 1) ((uint16_t*)w_out)[i] = ((const uint16_t*)w)[i];
                else ((float*)w_out)[i] = ((const float*)w)[i];
                continue;
            }
            const float r = fmaf(-a, load_x(grad, gdtype, i), wv);
            if (wdtype == 1) ((uint16_t*)w_out)[i] = orc_bf16_from_f32(r);
            else ((float*)w_out)[i] = r;
        }
    }
    if (n_clipped) *n_clipped = clipped;
}

/* ------------------------------------------------------------------------
 * FP8 (E4M3) per-tensor simulated quantization.  [Qwen] section "3. QAD"
 * (the table of quantized components: attention projections FP8 W8A8, KV
 * cache FP8) and [Nano] "NVFP4-Format und warum es wichtig ist?" (FP8 KV
 * cache) name the format but not its scaling; the reading taken is one
 * FP32 scale per tensor mapping the tensor amax onto the E4M3 maximum:
 *   s    = amax/448 (1 for an all-zero tensor), or a given (frozen) s;
 *   code = signbit(x)<<7 | E4M3(fl(|x|/s))   (nearest even, saturating);
 *   y    = bf16(fl(dec(code) * s)).
 * ---------------------------------------------------------------------- */
void orc_fp8_quantize(const void* x, int dtype, int64_t n, const float* tscale_in,
                      uint8_t* codes, float* tscale, uint16_t* y)
{
    float s;
    if (tscale_in) {
        s = *tscale_in;
    } else {
        const float amax = orc_amax(x, dtype, n);
        s = amax > 0.0f ? amax / 448.0f : 1.0f;
    }
    if (tscale) *tscale = s;
    for (int64_t i = 0; i < n; ++i) {
        const float v = load_x(x, dtype, i);
        const float q = fabsf(v) / s;
        const uint8_t c = (uint8_t)(orc_e4m3_encode(q) | (signbit(v) ? 0x80 : 0x00));
        if (codes) codes[i] = c;
        if (y) y[i] = orc_bf16_from_f32(orc_e4m3_decode(c) * s);
    }
}

/* ------------------------------------------------------------------------
 * MSE calibration (frozen-scale variant, [Lightning] section "量化尺度处理策略":
 * the MSE search is too expensive to redo every step, so its scales are
 * calibrated once and then kept fixed while only the weights train).
 * Candidates: block scale amax_b * k / 6 for n values of k spread evenly over
 * [k_min, k_max] (each k the binary32 value nearest the exact grid point).
 * Each candidate is rounded to E4M3 like a dynamic scale; its error is the
 * sum over the block, in element order, of the binary32 squares of
 * (x - dequantized fp32 value).  The first candidate with strictly smaller
 * error wins.  The tensor scale is the dynamic one and is frozen with them.
 * ---------------------------------------------------------------------- */
void orc_mse_kgrid(int n, float k_min, float k_max, float* k_out)
{
    for (int i = 0; i < n; ++i) {
        if (n == 1) { k_out[i] = k_min; continue; }
        double num = (double)k_min * (double)(n - 1 - i) + (double)k_max * (double)i;
        k_out[i] = (float)(num / (double)(n - 1));
    }
}

static float block_sq_error(const float* xb, float s_eff)
{
    uint8_t c16[16];
    float err = 0.0f;
    for (int j = 0; j < 16; ++j) {
        if (s_eff == 0.0f) c16[j] = 0;
        else c16[j] = orc_e2m1_encode(xb[j] / s_eff);
        float deq = orc_e2m1_decode(c16[j]) * s_eff;
        float d = xb[j] - deq;
        float sq = d * d;
        err = err + sq;
    }
    return err;
}

/* the n_cand values of k (any n_cand >= 1; the caller frees them) */
static float* cand_grid(int n_cand, float k_min, float k_max)
{
    float* k = (float*)malloc(sizeof(float) * (size_t)(n_cand > 0 ? n_cand : 1));
    if (!k) {
        fprintf(stderr, "oracle: no memory for %d MSE candidates\n", n_cand);
        abort();
    }
    orc_mse_kgrid(n_cand, k_min, k_max, k);
    return k;
}

static uint8_t calibrate_one_block(const float* xb, float s_g, int n_cand,
                                   const float* k, float* best_err,
                                   uint8_t* cand_codes, float* cand_err)
{
    float amax_b = 0.0f;
    for (int j = 0; j < 16; ++j) { float a = fabsf(xb[j]); if (a > amax_b) amax_b = a; }
    uint8_t best = 0;
    float best_e = INFINITY;
    for (int i = 0; i < n_cand; ++i) {
        float scaled = amax_b * k[i];
        uint8_t sb = block_scale_code(scaled, s_g);
        float s_eff = orc_e4m3_decode(sb) * s_g;
        float e = block_sq_error(xb, s_eff);
        if (cand_codes) cand_codes[i] = sb;
        if (cand_err) cand_err[i] = e;
        if (e < best_e) { best_e = e; best = sb; }
    }
    if (best_err) *best_err = best_e;
    return best;
}

void orc_mse_calibrate_blocks(const float* blocks, int64_t nblocks, float s_g,
                              int n_cand, float k_min, float k_max,
                              uint8_t* scales, float* err_out,
                              uint8_t* cand_codes, float* cand_err)
{
    float* k = cand_grid(n_cand, k_min, k_max);
    for (int64_t b = 0; b < nblocks; ++b) {
        float e;
        uint8_t sb = calibrate_one_block(blocks + b * 16, s_g, n_cand, k, &e,
                                         cand_codes ? cand_codes + b * n_cand : NULL,
                                         cand_err ? cand_err + b * n_cand : NULL);
        if (scales) scales[b] = sb;
        if (err_out) err_out[b] = e;
    }
    free(k);
}

void orc_mse_calibrate(const void* x, int dtype, int64_t R, int64_t C,
                       int n_cand, float k_min, float k_max,
                       uint8_t* scales, float* tscale)
{
    const int64_t n = R * C, nb = n / 16;
    float s_g = orc_tensor_scale(orc_amax(x, dtype, n));
    if (tscale) *tscale = s_g;
    float* k = cand_grid(n_cand, k_min, k_max);
    float xb[16];
    for (int64_t b = 0; b < nb; ++b) {
        for (int j = 0; j < 16; ++j) xb[j] = load_x(x, dtype, b * 16 + j);
        scales[b] = calibrate_one_block(xb, s_g, n_cand, k, NULL, NULL, NULL);
    }
    free(k);
}

/* ------------------------------------------------------------------------
 * KL distillation loss ([Nano] section "Von QAT zu QAD": the student is
 * trained to minimise the KL divergence to the frozen teacher's output token
 * distribution; [Qwen] section "3. QAD": the loss compares the two logit
 * vectors element by element over the vocabulary).
 * Readings: p = softmax(teacher/T), q = softmax(student/T),
 *   KL_row = sum_v p_v (log p_v - log q_v)   (forward KL, teacher first),
 *   loss   = mean over rows,
 *   dloss/ds_v scaled by grad_scale: (q_v - p_v) * grad_scale / T.
 * Binary64 with the usual max subtraction.  With d_v = log p_v - log q_v =
 * (t_v - s_v)/T - (LSE_t - LSE_s) we have q_v = p_v e^-d_v, so
 *   q_v - p_v = p_v expm1(-d_v),
 *   KL_row    = sum_v p_v (expm1(-d_v) + d_v),
 * the second because sum_v (q_v - p_v) = 0.  Every term of that sum is
 * non-negative, so binary64 keeps its relative accuracy however small the
 * divergence, and an error in the row constant LSE_t - LSE_s enters only to
 * second order; the plain sum of p_v d_v loses ~1e-14 nats to the rounding
 * of the log-normalisers, which is all of a divergence near 1e-10.
 * ---------------------------------------------------------------------- */
static double load_d(const void* p, int dtype, int64_t i)
{
    return (double)load_x(p, dtype, i);
}

double orc_kl_fwd_bwd(const void* teacher, const void* student, int dtype,
                      int64_t rows, int64_t V, double T, double grad_scale,
                      double* row_kl, double* grad)
{
    double total = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t o = r * V;
        double mt = -INFINITY, ms = -INFINITY;
        for (int64_t v = 0; v < V; ++v) {
            double t = load_d(teacher, dtype, o + v) / T;
            double s = load_d(student, dtype, o + v) / T;
            if (t > mt) mt = t;
            if (s > ms) ms = s;
        }
        double zt = 0.0, zs = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            zt += exp(load_d(teacher, dtype, o + v) / T - mt);
            zs += exp(load_d(student, dtype, o + v) / T - ms);
        }
        const double delta = (mt - ms) + log(zt / zs);   /* LSE_t - LSE_s */
        double kl = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            double t = load_d(teacher, dtype, o + v) / T;
            double s = load_d(student, dtype, o + v) / T;
            double d = (t - s) - delta;                     /* log p_v - log q_v */
            double p = exp(t - mt) / zt;
            double em = expm1(-d);                          /* q_v / p_v - 1 */
            kl += p * (em + d);
            if (grad) grad[o + v] = p * em * grad_scale / T;
        }
        if (row_kl) row_kl[r] = kl;
        total += kl;
    }
    return rows > 0 ? total / (double)rows : 0.0;
}

/* ------------------------------------------------------------------------
 * The same KL loss and gradient evaluated in binary32 (expf, logf, expm1f),
 * row by row in the order above.  TIMING VARIANT ONLY: it gives a CPU rate
 * in the arithmetic width the GPU kernels use; no parity test compares
 * against it (the binary64 function above is the reference).  Its test holds
 * it to the binary64 result within binary32 accuracy.
 * ---------------------------------------------------------------------- */
float orc_kl_fwd_bwd_f32(const void* teacher, const void* student, int dtype,
                         int64_t rows, int64_t V, float T, float grad_scale,
                         float* row_kl, float* grad)
{
    double total = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t o = r * V;
        float mt = -INFINITY, ms = -INFINITY;
        for (int64_t v = 0; v < V; ++v) {
            float t = load_x(teacher, dtype, o + v) / T;
            float s = load_x(student, dtype, o + v) / T;
            if (t > mt) mt = t;
            if (s > ms) ms = s;
        }
        float zt = 0.0f, zs = 0.0f;
        for (int64_t v = 0; v < V; ++v) {
            zt += expf(load_x(teacher, dtype, o + v) / T - mt);
            zs += expf(load_x(student, dtype, o + v) / T - ms);
        }
        const float delta = (mt - ms) + logf(zt / zs);
        float kl = 0.0f;
        for (int64_t v = 0; v < V; ++v) {
            float t = load_x(teacher, dtype, o + v) / T;
            float s = load_x(student, dtype, o + v) / T;
            float d = (t - s) - delta;
            float p = expf(t - mt) / zt;
            float em = expm1f(-d);
            kl += p * (em + d);
            if (grad) grad[o + v] = p * em * grad_scale / T;
        }
        if (row_kl) row_kl[r] = kl;
        total += kl;
    }
    return rows > 0 ? (float)(total / (double)rows) : 0.0f;
}

/* ------------------------------------------------------------------------
 * Teacher-top-k KL ([Qwen] "3. QAD": the distillation run restricts the KD
 * loss to the teacher's top-4096 vocabulary entries so that dense
 * [seq, vocab] logits need not exist).  The page gives neither the selection
 * rule at ties nor the normalisation; the reading taken:
 *   tau = the k-th largest teacher logit of the row (k >= V: every entry);
 *   S   = { v : t_v >= tau }   (every entry tied with tau is kept, so |S| >= k);
 *   p~, q~ = softmax(t/T), softmax(s/T) renormalised over S;
 *   row loss = sum_{v in S} p~_v (log p~_v - log q~_v);
 *   gradient = (q~_v - p~_v) * grad_scale / T on S, 0 elsewhere.
 * Binary64, evaluated as the full-vocabulary KL above (non-negative terms);
 * a sorted copy of the row gives tau.
 * ---------------------------------------------------------------------- */
static int cmp_desc(const void* a, const void* b)
{
    const double x = *(const double*)a, y = *(const double*)b;
    return x < y ? 1 : x > y ? -1 : 0;
}

/* KL of one row restricted to S = { v : t_v >= tau }, both softmaxes
 * renormalised over S; gradient 0 outside S.  Returns the row loss. */
static double kl_kept_row(const void* teacher, const void* student, int dtype, int64_t o, int64_t V,
                          double tau, double T, double grad_scale, double* grad, int64_t* count_out)
{
    double mt = -INFINITY, ms = -INFINITY;
    int64_t count = 0;
    for (int64_t v = 0; v < V; ++v) {
        const double tv = load_d(teacher, dtype, o + v);
        if (!(tv >= tau)) continue;
        ++count;
        const double t = tv / T, s = load_d(student, dtype, o + v) / T;
        if (t > mt) mt = t;
        if (s > ms) ms = s;
    }
    double zt = 0.0, zs = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        if (!(load_d(teacher, dtype, o + v) >= tau)) continue;
        zt += exp(load_d(teacher, dtype, o + v) / T - mt);
        zs += exp(load_d(student, dtype, o + v) / T - ms);
    }
    const double delta = (mt - ms) + log(zt / zs);   /* LSE_t - LSE_s over S */
    double kl = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        const double tv = load_d(teacher, dtype, o + v);
        if (!(tv >= tau)) {
            if (grad) grad[o + v] = 0.0;
            continue;
        }
        const double t = tv / T, s = load_d(student, dtype, o + v) / T;
        const double d = (t - s) - delta;
        const double p = exp(t - mt) / zt;
        const double em = expm1(-d);
        kl += p * (em + d);
        if (grad) grad[o + v] = p * em * grad_scale / T;
    }
    if (count_out) *count_out = count;
    return kl;
}

double orc_kl_topk_fwd_bwd(const void* teacher, const void* student, int dtype,
                           int64_t rows, int64_t V, int64_t k, double T, double grad_scale,
                           double* row_kl, double* grad, int64_t* row_count)
{
    double total = 0.0;
    double* sorted = (double*)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
    if (!sorted) return NAN;
    const int64_t kk = k < V ? k : V;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t o = r * V;
        for (int64_t v = 0; v < V; ++v) sorted[v] = load_d(teacher, dtype, o + v);
        qsort(sorted, (size_t)V, sizeof(double), cmp_desc);
        const double tau = sorted[kk - 1];
        const double kl = kl_kept_row(teacher, student, dtype, o, V, tau, T, grad_scale, grad,
                                      row_count ? row_count + r : NULL);
        if (row_kl) row_kl[r] = kl;
        total += kl;
    }
    free(sorted);
    return rows > 0 ? total / (double)rows : 0.0;
}

/* ------------------------------------------------------------------------
 * Teacher-top-p (nucleus) KL.  [Qwen] "3. QAD" names top-p as the variant to
 * try after the top-k run, without defining it; the reading taken is the
 * usual nucleus of the teacher distribution:
 *   p = softmax(t/T) over the whole row;
 *   walking the distinct teacher values from the largest down, accumulate
 *   the mass of every entry equal to each; tau = the first value at which
 *   the accumulated mass reaches top_p (top_p >= 1: every entry);
 *   S = { v : t_v >= tau } (ties with tau kept), then exactly as top-k.
 * Optional row_tau[rows]; row_mass[2*rows] = (mass strictly above tau, mass
 * at or above tau), which bound the decision's margin.
 * ---------------------------------------------------------------------- */
double orc_kl_topp_fwd_bwd(const void* teacher, const void* student, int dtype,
                           int64_t rows, int64_t V, double top_p, double T, double grad_scale,
                           double* row_kl, double* grad, int64_t* row_count, double* row_tau,
                           double* row_mass)
{
    double total = 0.0;
    double* sorted = (double*)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
    if (!sorted) return NAN;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t o = r * V;
        double mt = -INFINITY;
        for (int64_t v = 0; v < V; ++v) {
            sorted[v] = load_d(teacher, dtype, o + v);
            if (sorted[v] / T > mt) mt = sorted[v] / T;
        }
        double zt = 0.0;
        for (int64_t v = 0; v < V; ++v) zt += exp(sorted[v] / T - mt);
        qsort(sorted, (size_t)V, sizeof(double), cmp_desc);
        double tau = sorted[V - 1], above = 0.0, incl = 0.0;
        if (top_p < 1.0) {
            int64_t i = 0;
            while (i < V) {
                const double val = sorted[i];
                double m = 0.0;
                while (i < V && sorted[i] == val) m += exp(sorted[i++] / T - mt) / zt;
                above = incl;
                incl += m;
                tau = val;
                if (incl >= top_p) break;
            }
        } else {
            for (int64_t v = 0; v < V; ++v) incl += exp(sorted[v] / T - mt) / zt;
            above = incl - exp(sorted[V - 1] / T - mt) / zt;
        }
        const double kl = kl_kept_row(teacher, student, dtype, o, V, tau, T, grad_scale, grad,
                                      row_count ? row_count + r : NULL);
        if (row_kl) row_kl[r] = kl;
        if (row_tau) row_tau[r] = tau;
        if (row_mass) { row_mass[2 * r] = above; row_mass[2 * r + 1] = incl; }
        total += kl;
    }
    free(sorted);
    return rows > 0 ? total / (double)rows : 0.0;
}
