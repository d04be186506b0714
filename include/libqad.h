/*
 * libqad -- the data-parallel hot path of quantization-aware distillation
 * (QAD) for AMD Instinct MI355X (gfx950): NVFP4 simulated quantization of
 * weights and activations in the student's forward pass (dynamic or frozen
 * MSE-calibrated scales) with a straight-through backward, and the
 * KL(teacher || student) distillation loss with its gradient over the
 * vocabulary.
 *
 * Pages the operations follow (cited by title and section):
 *  [Nano]      "NVIDIA AI bringt Nemotron-3-Nano-30B auf NVFP4 mit Quantization
 *              Conscious Distillation (QAD) ..." (chatgpz.de):
 *              "NVFP4-Format und warum es wichtig ist?" -- 4-bit floating-point
 *              values in blocks of 16, one E4M3 scale per block, one FP32
 *              scale per tensor; "Von QAT zu QAD" -- the student minimises the
 *              KL divergence to a frozen BF16 teacher's token distribution.
 *  [Lightning] "使用量化感知蒸馏技术构建Nemotron 3.5 Lightning NVFP4模型"
 *              (163.com): "QAD的工作原理" -- every student forward runs
 *              simulated quantization; "量化尺度处理策略" -- dynamic scales are
 *              recomputed each step, frozen scales come from an MSE search
 *              done once and stay fixed while only the weights train.
 *  [Qwen]      "Model-Optimizer 实战：用量化感知蒸馏（QAD）恢复 Qwen3.6-35B-A3B 的
 *              W4A4 NVFP4 精度" (nlpx.cn): "3. QAD" -- the KD loss compares
 *              teacher and student logits element-wise over the vocabulary;
 *              dense fp32 [seq, vocab] logits do not fit, so the loss must
 *              stream the logits.
 *
 * Numerics (what the pages leave open is fixed as follows, identically in the
 * CPU reference the library is tested against):
 *  - E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}; nearest value, ties to the even
 *    code index, magnitudes above 6 saturate; the code's sign is the sign bit
 *    of x (so -0 gives code 0x8).
 *  - E4M3 is the OCP "E4M3FN" encoding (bias 7, max 448, subnormals), round to
 *    nearest even, saturating at 448.
 *  - tensor scale s_g = amax/2688 (2688 = 6 * 448), or 1 for an all-zero
 *    tensor; block scale s_b = E4M3((amax_b/6)/s_g); effective scale
 *    s_eff = dec(s_b) * s_g; code = E2M1(x/s_eff) with the quotient correctly
 *    rounded to binary32 (a zero effective scale gives signed-zero codes);
 *    dequantized value y = bf16(dec(code) * s_eff).  Every operation is one
 *    IEEE binary32 operation rounded to nearest even, in that order.
 *  - Codes are packed two per byte, the even element in the low nibble,
 *    row-major [R][C/2]; block scales row-major [R][C/16]; blocks run along
 *    the contiguous last dimension.
 *  - KL: p = softmax(t/T), q = softmax(s/T), loss = mean over token rows of
 *    sum_v p_v (log p_v - log q_v) in nats; gradient w.r.t. the student logits
 *    = (q - p) * grad_scale / T.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or keeps them.  Scratch memory comes from the
 *    caller's `workspace` (size from qad_workspace_bytes(), 256-byte aligned;
 *    its contents need not be initialised and are overwritten).
 *  - All work is enqueued asynchronously on `stream` (0 = the null stream);
 *    the call returns once it is enqueued.
 *  - Arguments are checked on the host before anything is launched; a failed
 *    check returns its status and launches nothing.  A failed launch returns
 *    QAD_ERR_HIP.  Calls that share a workspace must not overlap in time.
 *  - Empty inputs are valid, and a pointer to an empty buffer may be NULL.
 *    For tensors with R*C == 0 nothing is coded;
 *    tscale_out (when given) receives 1.0f per tensor, the scale of the
 *    zero tensor, or with frozen scales the given tscale_in, and
 *    nvfp4_amax writes 0.  The KL losses with tokens == 0 write loss 0.
 *  - Inputs must be finite.  A NaN or infinity makes the tensor amax and the
 *    tensor scale non-finite (visible in amax_out / tscale_out, or through
 *    qad_check_finite()); the other outputs are then unspecified.
 *  - Alignment: tensor pointers 16-byte aligned, packed codes 4-byte aligned;
 *    scale and scalar pointers have no requirement beyond their type.
 *  - Results are deterministic: the same inputs give bitwise-equal outputs,
 *    in every process (every sum has a fixed order).
 *  - Thread-safe.  The state kept across calls: per device and written
 *    once, the compute-unit count, the quantizer's occupancy and the
 *    device address of nvfp4_quantize_noalloc's scratch (atomics);
 *    process-wide, the wait bound of qad_set_wait_limit_us (an atomic).
 *    Calls only enqueue kernels on `stream` (no memset, no allocation, no
 *    host synchronisation; qad_check_finite excepted), so a sequence of
 *    calls can be captured into a HIP graph.
 */
#ifndef LIBQAD_H
#define LIBQAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* qad_stream_t; /* the same handle as hipStream_t */

typedef enum {
    QAD_OK = 0,
    QAD_ERR_INVALID_ARG = 1, /* null pointer where one is required, bad enum, bad parameter */
    QAD_ERR_SHAPE = 2,       /* negative size, C not a multiple of 16, size overflow        */
    QAD_ERR_DTYPE = 3,       /* dtype not supported by this entry point                    */
    QAD_ERR_ALIGNMENT = 4,   /* pointer not aligned as the conventions above require       */
    QAD_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than qad_workspace_bytes()       */
    QAD_ERR_NONFINITE = 6,   /* qad_check_finite() found a NaN or infinity                 */
    QAD_ERR_HIP = 7          /* a HIP launch or copy failed                                */
} qad_status_t;

typedef enum { QAD_F32 = 0, QAD_BF16 = 1 } qad_dtype_t;

typedef enum {
    QAD_OP_AMAX = 0,          /* nvfp4_amax                                   */
    QAD_OP_QUANTIZE = 1,      /* nvfp4_quantize and nvfp4_qdq_fwd             */
    QAD_OP_MSE_CALIBRATE = 2, /* nvfp4_mse_calibrate                          */
    QAD_OP_KL = 3,            /* qad_kl_fwd_bwd: B = 1, R = tokens, C = vocab */
    QAD_OP_KL_TOPK = 4,       /* qad_kl_topk_fwd_bwd: B = 1, R = tokens, C = vocab */
    QAD_OP_W4A4_LINEAR = 5,   /* qad_w4a4_linear_fwd / _bwd: B = M, R = N, C = K */
    QAD_OP_KL_TOPP = 6        /* qad_kl_topp_fwd_bwd: B = 1, R = tokens, C = vocab */
} qad_op_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* qad_status_string(qad_status_t status);

/* Version of this ABI (incremented on any incompatible change). */
int qad_abi_version(void);

/* Bound on the device-side waits of the one-pass kernels, in microseconds of
 * wall clock (default 20000).  The dynamic quantizers (nvfp4_quantize,
 * nvfp4_qdq_fwd, fp8_quantize and the W4A4 linear when a tensor fits on chip)
 * and the KL segment kernels (rows of more than 16384 logits) exchange
 * partial results between workgroups that are resident together; a workgroup
 * whose wait reaches the bound computes what it waited for from the inputs
 * itself, with the same arithmetic, so results never depend on the bound --
 * only the time does, when other work keeps workgroups from being resident.
 * 0 makes every wait give up at once (which exercises those paths).  Applies
 * to calls made after it, process-wide; us < 0 only queries.  Returns the
 * previous bound.  Host-only, never fails. */
int64_t qad_set_wait_limit_us(int64_t us);

/* Bytes of workspace entry point `op` needs for B tensors of R x C elements
 * of either dtype (for QAD_OP_KL: R token rows of C vocabulary logits).
 * Always a multiple of 256.  Returns 0 for invalid sizes (the entry point
 * then reports the shape error).  Frozen-scale quantization needs none. */
size_t qad_workspace_bytes(qad_op_t op, int64_t B, int64_t R, int64_t C);

/* Tensor amax (max calibration, [Lightning] "量化尺度处理策略"): amax_out[b] =
 * max |x[b]| over each of B contiguous tensors of R x C elements.
 *   x         : device, dtype xt (QAD_F32 or QAD_BF16), [B][R][C], 16-byte
 *               aligned; C * sizeof(dtype) must be a multiple of 16
 *   amax_out  : device float[B]
 *   workspace : qad_workspace_bytes(QAD_OP_AMAX, B, R, C) bytes, 256-byte aligned */
qad_status_t nvfp4_amax(const void* x, qad_dtype_t xt, int64_t B, int64_t R, int64_t C,
                        float* amax_out, void* workspace, size_t ws_bytes, qad_stream_t stream);

/* NVFP4 quantization of B independent tensors [R][C] ([Nano] "NVFP4-Format
 * und warum es wichtig ist?"; dynamic vs frozen per [Lightning] "量化尺度处理策略").
 *   x          : device, dtype xt, [B][R][C], C % 16 == 0, 16-byte aligned
 *   scales_in  : NULL -> dynamic scales (amax, tensor scale and block scales
 *                computed from x on every call); non-NULL -> frozen scales:
 *                device u8 [B][R][C/16] E4M3 codes (0x00..0x7E), with
 *   tscale_in  : device float[B] frozen tensor scales (positive, finite);
 *                required iff scales_in is non-NULL
 *   codes      : device u8 [B][R][C/2] packed E2M1 codes, or NULL
 *   scales_out : device u8 [B][R][C/16] block scales used, or NULL
 *   tscale_out : device float[B] tensor scales used, or NULL
 *   y          : device bf16 [B][R][C] dequantized values, or NULL
 *   workspace  : device scratch of qad_workspace_bytes(QAD_OP_QUANTIZE, ...)
 * At least one output must be non-NULL.  x must not overlap any output. */
qad_status_t nvfp4_quantize(const void* x, qad_dtype_t xt, int64_t B, int64_t R, int64_t C,
                            const uint8_t* scales_in, const float* tscale_in,
                            uint8_t* codes, uint8_t* scales_out, float* tscale_out, void* y,
                            void* workspace, size_t ws_bytes, qad_stream_t stream);

/* nvfp4_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, outputs and errors without the workspace.  Dynamic
 * scales keep their tensor records in a fixed 16 MiB scratch array inside
 * the library (one per GPU, held until the process ends), so a call needs
 * qad_workspace_bytes(QAD_OP_QUANTIZE, B, R, C) <= 16 MiB (the 128-expert
 * 2048 x 4096 batch needs 9.5 MiB) and returns QAD_ERR_WORKSPACE beyond that;
 * frozen scales need no scratch.  The call allocates nothing (no hipMalloc,
 * no library allocation); it clears the records it uses on `stream` before
 * its kernels read them.  Every call on one GPU shares that GPU's scratch:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and give unspecified results -- order them on one stream, or use
 * nvfp4_quantize with workspaces of their own.  QAD_ERR_HIP if the scratch's
 * device address cannot be obtained. */
qad_status_t nvfp4_quantize_noalloc(const void* x, qad_dtype_t xt, int64_t B, int64_t R, int64_t C,
                                    const uint8_t* scales_in, const float* tscale_in,
                                    uint8_t* codes, uint8_t* scales_out, float* tscale_out, void* y,
                                    qad_stream_t stream);

/* Simulated quantization forward (quantize + dequantize, "QDQ") as run in
 * every student forward pass ([Lightning] "QAD的工作原理"): y = the
 * dequantized bf16 values of nvfp4_quantize, nothing else written. */
qad_status_t nvfp4_qdq_fwd(const void* x, qad_dtype_t xt, int64_t B, int64_t R, int64_t C,
                           const uint8_t* scales_in, const float* tscale_in, void* y,
                           void* workspace, size_t ws_bytes, qad_stream_t stream);

/* Straight-through backward of the QDQ: grad_x = grad_y bit for bit (the
 * rounding is treated as identity; scales receive no gradient because dynamic
 * scales are recomputed and frozen ones stay fixed, [Lightning] "量化尺度处理策略").
 *   grad_y, grad_x : device, n elements of dtype gt, 16-byte aligned;
 *   grad_x == grad_y is allowed (nothing is launched); partial overlap is not. */
qad_status_t nvfp4_qdq_bwd(const void* grad_y, void* grad_x, qad_dtype_t gt, int64_t n,
                           qad_stream_t stream);

/* Clipped straight-through backward ([Lightning] "量化尺度处理策略": with
 * frozen scales only the weights train; the pages print no clipping rule).
 * grad_x = grad_y bit for bit where |x| <= 6 * s_eff, the range the element's
 * block can represent, and +0 where the forward saturated; s_eff =
 * fl(dec(s_b) * s_g) is the forward's binary32 effective scale and the
 * comparison is exact.  The scales are the ones the forward used: the frozen
 * ones, or scales_out / tscale_out of a dynamic nvfp4_quantize.
 *   grad_y     : device, dtype gt, [B][R][C], 16-byte aligned
 *   x          : device, dtype xt, [B][R][C], 16-byte aligned (the forward input)
 *   scales     : device u8 [B][R][C/16] E4M3 block scale codes (0..126)
 *   tscale     : device float[B] tensor scales (positive, finite), 4-byte aligned
 *   grad_x     : device, dtype gt, [B][R][C], 16-byte aligned; grad_x == grad_y
 *                is allowed (in place); any other overlap with an input is not
 * C % 16 == 0.  Other scale codes or tensor scales give unspecified results. */
qad_status_t nvfp4_qdq_bwd_clipped(const void* grad_y, qad_dtype_t gt, const void* x, qad_dtype_t xt,
                                   int64_t B, int64_t R, int64_t C, const uint8_t* scales,
                                   const float* tscale, void* grad_x, qad_stream_t stream);

/* Frozen-scale SGD weight step, the clipped straight-through gradient fused
 * into the update ([Lightning] "量化尺度处理策略": with frozen scales the
 * scales stay fixed and only the weights are updated; "训练配置": a constant
 * learning rate and gradient clipping at norm 1.0).  The pages name no
 * optimizer; this is plain SGD, and the clipping coefficient
 * (min(1, max_norm / global gradient norm)) is the caller's, since it needs
 * every parameter's gradient.  With a = fl32(lr * clip_coef), element by
 * element:
 *   w_out = w                          where |w| > 6 * s_eff (the quantizer
 *                                      saturates: no gradient reaches w),
 *   w_out = round(fma32(-a, g, w))     elsewhere (one binary32 rounding, then
 *                                      nearest-even bf16 for bf16 weights),
 * with s_eff = fl(dec(s_b) * s_g) and the exact comparison of
 * nvfp4_qdq_bwd_clipped.  The weight is the forward's input, so one pass
 * reads w, g and the scales and writes w_out.
 *   w          : device, dtype wt, [B][R][C], 16-byte aligned, finite
 *   grad       : device, dtype gt, [B][R][C], 16-byte aligned (gradient of the
 *                loss wrt the QDQ output)
 *   scales     : device u8 [B][R][C/16] frozen E4M3 block scale codes (0..126)
 *   tscale     : device float[B] frozen tensor scales (positive, finite)
 *   lr, clip_coef : finite (QAD_ERR_INVALID_ARG otherwise)
 *   w_out      : device, dtype wt, [B][R][C], 16-byte aligned; w_out == w is
 *                allowed (in place); any other overlap with an input is not
 * C % 16 == 0.  Other scale codes or tensor scales give unspecified results. */
qad_status_t nvfp4_frozen_sgd_step(const void* w, qad_dtype_t wt, const void* grad, qad_dtype_t gt,
                                   int64_t B, int64_t R, int64_t C, const uint8_t* scales,
                                   const float* tscale, float lr, float clip_coef, void* w_out,
                                   qad_stream_t stream);

/* MSE calibration of the frozen block scales ([Lightning] "量化尺度处理策略":
 * the MSE scale search runs once, before training, because it is too costly
 * per step).  For each block the candidates are amax_b * k_i / 6 with k_i the
 * binary32 value nearest to k_min + (k_max - k_min) * i / (n - 1),
 * i = 0..n-1, each rounded to E4M3 like a dynamic scale; the error of a
 * candidate is sum_j (x_j - dequantized_j)^2 over the block in element order
 * (binary32, values before the bf16 rounding); the first candidate with
 * strictly smaller error wins.  The tensor scale is the dynamic one.
 *   w          : device, dtype wt, [B][R][C], C % 16 == 0, 16-byte aligned
 *   n_candidates >= 1, 0 < k_min <= k_max, and when n > 1
 *                (k_max - k_min) / (n - 1) <= k_min / 16 (consecutive
 *                candidates then never skip an E4M3 value, which the search
 *                relies on; the 64-candidate grid over [0.5, 1] qualifies)
 *   scales_out : device u8 [B][R][C/16]
 *   tscale_out : device float[B]
 * Feed scales_out / tscale_out to nvfp4_quantize / nvfp4_qdq_fwd as the
 * frozen scales. */
qad_status_t nvfp4_mse_calibrate(const void* w, qad_dtype_t wt, int64_t B, int64_t R, int64_t C,
                                 int32_t n_candidates, float k_min, float k_max,
                                 uint8_t* scales_out, float* tscale_out,
                                 void* workspace, size_t ws_bytes, qad_stream_t stream);

/* FP8 (OCP E4M3FN) per-tensor simulated quantization ([Qwen] "3. QAD": the
 * attention projections are kept in FP8 W8A8 and the KV cache in FP8; [Nano]:
 * FP8 KV cache).  The pages give no scaling rule; the one taken here is one
 * FP32 scale per tensor: s = amax/448 (1 for an all-zero tensor), or the
 * given frozen / static scale; code = sign(x) << 7 | E4M3(|x|/s) with the
 * quotient correctly rounded, nearest even, saturating at 448;
 * y = bf16(dec(code) * s).  The straight-through backward is nvfp4_qdq_bwd.
 *   x          : device, dtype xt, B tensors of R x C, C % 8 == 0
 *   tscale_in  : device float[B] frozen scales (> 0, finite), or NULL for
 *                dynamic scales (computed from each tensor's amax)
 *   codes      : device u8[B][R][C] (8-byte aligned), or NULL
 *   tscale_out : device float[B] scales used, or NULL
 *   y          : device bf16[B][R][C], or NULL (at least one output)
 *   workspace  : qad_workspace_bytes(QAD_OP_QUANTIZE, B, R, C) bytes for
 *                dynamic scales; unused (may be NULL) with tscale_in */
qad_status_t fp8_quantize(const void* x, qad_dtype_t xt, int64_t B, int64_t R, int64_t C,
                          const float* tscale_in, uint8_t* codes, float* tscale_out, void* y,
                          void* workspace, size_t ws_bytes, qad_stream_t stream);

/* Bytes of a packed NVFP4 tensor of R x C elements (C % 16 == 0), the
 * W4A4 linear's saved operand form: the E2M1 codes (R*C/2 bytes, row-major,
 * even element in the low nibble), then the E4M3 block scales (R*C/16 bytes,
 * row-major) at byte R*C/2, then the fp32 tensor scale at the next multiple
 * of 16 bytes; the padding before and after the tensor scale is never
 * written.  0 for invalid sizes. */
size_t qad_nvfp4_packed_bytes(int64_t R, int64_t C);

/* W4A4 NVFP4 fake-quant linear layer ([Qwen] "3. QAD": the student is the
 * W4A4 NVFP4 model, weights and activations both NVFP4; [Lightning]
 * "QAD的工作原理": simulated quantization in every student forward).
 *   forward : y[M][N] = QDQ(x)[M][K] * QDQ(w)[N][K]^T, where QDQ is
 *             nvfp4_qdq_fwd (blocks of 16 along K): dynamic scales for x;
 *             for w dynamic scales too, or the frozen ones given
 *             ([Lightning] "量化尺度处理策略": frozen-scale QAD keeps the
 *             MSE-calibrated weight scales fixed while the weights train);
 *             each output is the bf16 rounding of an fp32 sum of the bf16
 *             QDQ values' products.  x and w are quantized once each into
 *             packed NVFP4 operands (qad_nvfp4_packed_bytes); the product
 *             reads those and rebuilds the bf16 QDQ values on chip (the
 *             library's own MFMA kernel; no other library is called and the
 *             call never synchronises).
 *   x, w    : device, dtype dt, row-major, 16-byte aligned; K > 0, K % 16 == 0
 *   w_scales_in, w_tscale_in : device u8 [N][K/16] and float[1], frozen
 *             scales of w (as from nvfp4_mse_calibrate), or both NULL
 *   y       : device bf16 [M][N]
 *   xq, wq  : device, qad_nvfp4_packed_bytes(M, K) and (N, K) bytes, 16-byte
 *             aligned: receive the packed NVFP4 forms of x and w (kept for the
 *             backward); no output may overlap another or an input
 *   workspace : qad_workspace_bytes(QAD_OP_W4A4_LINEAR, M, N, K) bytes (the
 *             quantizer's records)
 * M == 0 or N == 0: y is empty and the other operand's packed form (xq or
 * wq) is still written; pointers of empty buffers may be NULL.  The fp32
 * sums are formed in a fixed order, so results are reproducible bit for bit. */
qad_status_t qad_w4a4_linear_fwd(const void* x, const void* w, qad_dtype_t dt, int64_t M, int64_t N, int64_t K,
                                 const uint8_t* w_scales_in, const float* w_tscale_in, void* y, void* xq, void* wq,
                                 void* workspace, size_t ws_bytes, qad_stream_t stream);

/* Backward of qad_w4a4_linear_fwd with the straight-through estimator through
 * both quantizers: grad_x[M][K] = grad_y[M][N] * QDQ(w)[N][K] and
 * grad_w[N][K] = grad_y^T * QDQ(x)[M][K] (bf16 of fp32 sums), QDQ(x), QDQ(w)
 * rebuilt on chip from the forward's packed operands.
 *   grad_y : device bf16 [M][N], 16-byte aligned; xq, wq: the forward's
 *            packed operands
 *   grad_x, grad_w : device bf16 outputs, either may be NULL (not both,
 *                    unless both are empty)
 *   workspace, ws_bytes : unused (may be NULL / 0)
 * M == 0 or N == 0 writes zeros to the other gradient. */
qad_status_t qad_w4a4_linear_bwd(const void* grad_y, const void* xq, const void* wq, int64_t M, int64_t N, int64_t K,
                                 void* grad_x, void* grad_w, void* workspace, size_t ws_bytes, qad_stream_t stream);

/* Fused KL(teacher || student) forward + backward over the full vocabulary
 * ([Nano] "Von QAT zu QAD"; [Qwen] "3. QAD").
 *   teacher, student : device, dtype lt, [tokens][vocab] row-major, 16-byte
 *                      aligned, vocab % 8 == 0
 *   temperature      : T > 0 (finite)
 *   grad_scale       : multiplies the gradient (1/tokens for the mean loss)
 *   loss_out         : device float[1]: mean over rows of the per-row KL (nats)
 *   row_loss         : device float[tokens] per-row KL, or NULL
 *   grad_student     : device [tokens][vocab] of dtype gt (QAD_BF16, or
 *                      QAD_F32 for full-precision gradients), or NULL for
 *                      the forward only; must not overlap the inputs
 *   workspace        : qad_workspace_bytes(QAD_OP_KL, 1, tokens, vocab) bytes
 *                      (per-row exchange records, partial sums of the
 *                      mean; per-row losses when row_loss is NULL) */
qad_status_t qad_kl_fwd_bwd(const void* teacher, const void* student, qad_dtype_t lt,
                            int64_t tokens, int64_t vocab, float temperature, float grad_scale,
                            float* loss_out, float* row_loss, void* grad_student, qad_dtype_t gt,
                            void* workspace, size_t ws_bytes, qad_stream_t stream);

/* Teacher-top-k KL forward + backward ([Qwen] "3. QAD": the distillation run
 * restricts the KD loss to the teacher's top-4096 vocabulary entries; the page
 * gives neither the tie rule nor the normalisation).  Per token row:
 *   tau = the k-th largest teacher logit (k >= vocab: the smallest);
 *   S   = every entry with teacher logit >= tau (entries tied with tau are all
 *         kept, so |S| >= min(k, vocab); -0 and +0 count as equal);
 *   loss = KL(p~ || q~) with p~, q~ = softmax(t/T), softmax(s/T) renormalised
 *          over S; gradient (q~ - p~) * grad_scale / T on S and exactly 0
 *          elsewhere.
 * Arguments as qad_kl_fwd_bwd, plus
 *   k         : >= 1
 *   workspace : qad_workspace_bytes(QAD_OP_KL_TOPK, 1, tokens, vocab) bytes
 *               (the qad_kl_fwd_bwd workspace followed by one float per row
 *               for the thresholds) */
qad_status_t qad_kl_topk_fwd_bwd(const void* teacher, const void* student, qad_dtype_t lt,
                                 int64_t tokens, int64_t vocab, int64_t k, float temperature,
                                 float grad_scale, float* loss_out, float* row_loss, void* grad_student,
                                 qad_dtype_t gt, void* workspace, size_t ws_bytes, qad_stream_t stream);

/* Teacher-top-p (nucleus) KL forward + backward ([Qwen] "3. QAD" names top-p
 * as the variant to try after the top-k run; no definition is printed).  Per
 * token row, with p = softmax(teacher/T) over the whole row:
 *   tau = the largest teacher value at which the teacher mass of the entries
 *         at or above it reaches top_p (top_p >= 1: the smallest value);
 *   S   = { v : teacher_v >= tau } (ties with tau kept; -0 equals +0);
 *   then exactly as qad_kl_topk_fwd_bwd on S.
 * The masses are the exponentials the KL kernels use, summed exactly in
 * 64-bit fixed point (2^-40 of the row's largest weight), so the choice is
 * deterministic; where the accumulated mass lies within about 1e-6 of top_p
 * it may differ from an exact-arithmetic choice by one group of tied values.
 *   top_p            : > 0 and finite
 *   tau_out          : device float[tokens] thresholds, or NULL; must not
 *                      overlap any other argument
 *   workspace        : qad_workspace_bytes(QAD_OP_KL_TOPP, 1, tokens, vocab)
 * Other arguments, layouts and errors as qad_kl_topk_fwd_bwd. */
qad_status_t qad_kl_topp_fwd_bwd(const void* teacher, const void* student, qad_dtype_t lt, int64_t tokens,
                                 int64_t vocab, float top_p, float temperature, float grad_scale, float* loss_out,
                                 float* row_loss, void* grad_student, qad_dtype_t gt, float* tau_out,
                                 void* workspace, size_t ws_bytes, qad_stream_t stream);

/* Synchronises `stream`, copies n floats from device memory `values` (an
 * amax_out or tscale_out array) and returns QAD_ERR_NONFINITE if any is a NaN
 * or an infinity, QAD_OK otherwise.  The only blocking call of the library. */
qad_status_t qad_check_finite(const float* values, int64_t n, qad_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBQAD_H */
