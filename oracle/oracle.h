/*
 * CPU oracle for the QAD hot path: NVFP4 simulated quantization and the
 * KL(teacher || student) distillation loss.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code with the HIP
 * library: it is written from the pages' definitions, slow and plain on
 * purpose, single-threaded.
 *
 * Pages cited (by title):
 *  [Nano]      "NVIDIA AI bringt Nemotron-3-Nano-30B auf NVFP4 mit Quantization
 *              Conscious Distillation (QAD) fuer effiziente Argumentationsinferenz"
 *              (chatgpz.de) -- sections "NVFP4-Format und warum es wichtig ist?",
 *              "Von QAT zu QAD", "Wichtige Erkenntnisse".
 *  [Lightning] "使用量化感知蒸馏技术构建Nemotron 3.5 Lightning NVFP4模型"
 *              (163.com) -- sections "QAD的工作原理", "量化尺度处理策略".
 *  [Qwen]      "Model-Optimizer 实战：用量化感知蒸馏（QAD）恢复 Qwen3.6-35B-A3B 的
 *              W4A4 NVFP4 精度" (nlpx.cn) -- section "3. QAD".
 *
 * The pages fix the format (16-element blocks, an E4M3 scale per block, an FP32
 * scale per tensor, 4-bit floating-point values), the two scale policies
 * (dynamic / frozen MSE-calibrated) and the loss (KL divergence to a frozen
 * teacher over the vocabulary).  Everything they leave open (grid, scale
 * formulas, rounding, layouts, KL direction/reduction) is fixed by the reading
 * stated next to the code that takes it, in oracle.c.
 *
 * Precision: the quantizer is defined in IEEE binary32 with round-to-nearest-
 * even for every operation (the tensor scale is FP32 per [Nano]); the KL loss
 * and gradient are computed in binary64.
 *
 * Parity status: every function here is pinned by CPU tests against closed
 * forms, exhaustive library cross-checks, invariants or hand-derived fixtures.
 */
#ifndef QAD_ORACLE_H
#define QAD_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar codecs ---------------------------------------------------- */
uint8_t  orc_e2m1_encode(float r);            /* 4-bit code sign<<3 | idx       */
float    orc_e2m1_decode(uint8_t code);       /* signed grid value              */
uint8_t  orc_e4m3_encode(float v);            /* v >= 0 finite, saturating      */
float    orc_e4m3_decode(uint8_t code);
uint16_t orc_bf16_from_f32(float f);          /* round-to-nearest-even          */
float    orc_f32_from_bf16(uint16_t h);

/* array forms of the codecs (for exhaustive tests) */
void orc_e2m1_encode_array(const float* r, int64_t n, uint8_t* out);
void orc_e4m3_encode_array(const float* v, int64_t n, uint8_t* out);
void orc_bf16_from_f32_array(const float* f, int64_t n, uint16_t* out);

/* ---- NVFP4 tensor operations ------------------------------------------ */
/* dtype of an input tensor: 0 = fp32, 1 = bf16 (raw 16-bit patterns)      */
float orc_amax(const void* x, int dtype, int64_t n);

/* Quantize one tensor [R][C] (C % 16 == 0).
 *   scales_in == NULL : dynamic scales (amax -> tensor scale -> block scales)
 *   scales_in != NULL : frozen scales; *tscale_in is the tensor scale
 * Outputs (each may be NULL): codes u8[R][C/2] (low nibble = even element),
 * scales u8[R][C/16] (E4M3), *tscale (fp32), y bf16[R][C] (dequantized).   */
void orc_nvfp4_quantize(const void* x, int dtype, int64_t R, int64_t C,
                        const uint8_t* scales_in, const float* tscale_in,
                        uint8_t* codes, uint8_t* scales, float* tscale,
                        uint16_t* y);

/* The blocks of a tensor are independent once its tensor scale s_g is known:
 * quantize nblocks consecutive 16-element blocks of x under s_g (dynamic block
 * scales, or frozen ones from scales_in).  Used to check samples of tensors
 * too large to quantize whole on the CPU. */
void orc_nvfp4_quantize_blocks(const void* x, int dtype, int64_t nblocks, float s_g,
                               const uint8_t* scales_in, uint8_t* codes, uint8_t* scales,
                               uint16_t* y);

/* Tensor scale from an amax. */
float orc_tensor_scale(float amax);

/* The k_i grid of the MSE search: n values in [k_min, k_max]. */
void orc_mse_kgrid(int n, float k_min, float k_max, float* k_out);

/* MSE calibration of one tensor: writes E4M3 block scales and the (frozen)
 * tensor scale.                                                             */
void orc_mse_calibrate(const void* x, int dtype, int64_t R, int64_t C,
                       int n_cand, float k_min, float k_max,
                       uint8_t* scales, float* tscale);

/* MSE calibration of a list of single 16-element blocks under a given tensor
 * scale (the blocks are independent once the tensor scale is known).
 * blocks: fp32 [nblocks][16].  Optional err_out: fp32 [nblocks] best error;
 * optional cand_codes: u8 [nblocks][n_cand] the E4M3 code of every candidate;
 * optional cand_err: fp32 [nblocks][n_cand] every candidate's error.        */
void orc_mse_calibrate_blocks(const float* blocks, int64_t nblocks, float s_g,
                              int n_cand, float k_min, float k_max,
                              uint8_t* scales, float* err_out,
                              uint8_t* cand_codes, float* cand_err);

/* ---- clipped straight-through backward --------------------------------
 * One tensor of nblocks 16-element blocks with the forward's block scales
 * and tensor scale s_g: grad_x = grad_y where |x| <= 6 * dec(s_b) * s_g
 * (exact), +0 elsewhere.  grad in gdtype, x in xdtype (0 fp32, 1 bf16).
 * Optional n_clipped: number of zeroed elements.                          */
void orc_nvfp4_qdq_bwd_clipped(const void* grad_y, int gdtype, const void* x, int xdtype,
                               int64_t nblocks, const uint8_t* scales, float s_g,
                               void* grad_x, int64_t* n_clipped);

/* ---- frozen-scale SGD weight step --------------------------------------
 * w' = w where |w| > 6 dec(scales[b]) s_g, else round_w(fmaf(-fl32(lr *
 * clip_coef), g, w)); w and w_out (may alias) of dtype wdtype, grad of
 * gdtype (0 = float32, 1 = bf16 bits).  Optional n_clipped: weights the clip
 * left unchanged. */
void orc_nvfp4_frozen_sgd_step(const void* w, int wdtype, const void* grad, int gdtype, int64_t nblocks,
                               const uint8_t* scales, float s_g, float lr, float clip_coef, void* w_out,
                               int64_t* n_clipped);

/* ---- FP8 (E4M3) per-tensor QDQ ---------------------------------------------
 * x: n elements of dtype.  tscale_in NULL: dynamic s = amax/448 (1 for an
 * all-zero tensor); else s = *tscale_in (> 0).  Optional codes[n] (E4M3 with
 * the sign of x in bit 7), tscale[1], y[n] (bf16 bits).                    */
void orc_fp8_quantize(const void* x, int dtype, int64_t n, const float* tscale_in,
                      uint8_t* codes, float* tscale, uint16_t* y);

/* ---- KL(teacher || student) ---------------------------------------------
 * teacher, student: [rows][V] in dtype (0 fp32, 1 bf16).
 * Writes row_kl[rows] (binary64, nats), optional grad[rows][V] (binary64) =
 * (softmax(s/T) - softmax(t/T)) * grad_scale / T.  Returns the mean loss.  */
double orc_kl_fwd_bwd(const void* teacher, const void* student, int dtype,
                      int64_t rows, int64_t V, double T, double grad_scale,
                      double* row_kl, double* grad);

/* ---- binary32 KL (timing variant, not a parity reference) --------------- */
float orc_kl_fwd_bwd_f32(const void* teacher, const void* student, int dtype,
                         int64_t rows, int64_t V, float T, float grad_scale,
                         float* row_kl, float* grad);

/* ---- teacher-top-k KL -----------------------------------------------------
 * As orc_kl_fwd_bwd restricted to S = { v : t_v >= k-th largest teacher logit
 * of the row } (ties kept), both distributions renormalised over S; gradient
 * 0 outside S.  Optional row_count[rows] = |S|.  k >= 1.                    */
double orc_kl_topk_fwd_bwd(const void* teacher, const void* student, int dtype,
                           int64_t rows, int64_t V, int64_t k, double T, double grad_scale,
                           double* row_kl, double* grad, int64_t* row_count);

/* ---- teacher-top-p (nucleus) KL -------------------------------------------
 * As orc_kl_topk_fwd_bwd with tau = the largest teacher value at which the
 * teacher mass of the entries at or above it reaches top_p (ties kept;
 * top_p >= 1: every entry).  Optional row_tau[rows] (the threshold) and
 * row_mass[2*rows] (mass strictly above tau, mass at or above tau).        */
double orc_kl_topp_fwd_bwd(const void* teacher, const void* student, int dtype,
                           int64_t rows, int64_t V, double top_p, double T, double grad_scale,
                           double* row_kl, double* grad, int64_t* row_count, double* row_tau,
                           double* row_mass);

/* ---- all-cores harness (oracle_omp.c; benchmark CPU baseline only) -------
 * The functions above, run with OpenMP over tensors, rows or row ranges;
 * results equal the single-threaded calls bit for bit. */
int    orc_omp_threads(void);
void   orc_omp_quantize_batch(const void* x, int dtype, int64_t B, int64_t R, int64_t C,
                              uint8_t* codes, uint8_t* scales, float* tscale, uint16_t* y);
void   orc_omp_quantize_tensor(const void* x, int dtype, int64_t R, int64_t C, const uint8_t* scales_in,
                               const float* tscale_in, uint8_t* codes, uint8_t* scales, float* tscale,
                               uint16_t* y);
void   orc_omp_mse_calibrate(const void* x, int dtype, int64_t R, int64_t C, int n_cand, float k_min,
                             float k_max, uint8_t* scales, float* tscale);
double orc_omp_kl_fwd_bwd(const void* teacher, const void* student, int dtype, int64_t rows, int64_t V,
                          double T, double grad_scale, double* row_kl, double* grad);
float  orc_omp_kl_fwd_bwd_f32(const void* teacher, const void* student, int dtype, int64_t rows, int64_t V,
                              float T, float grad_scale, float* row_kl, float* grad);

#ifdef __cplusplus
}
#endif
#endif
