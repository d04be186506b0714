// C-ABI entry points of libqad: argument validation, workspace layout and
// launch sequencing.  Declarations, ownership and error rules:
// include/libqad.h.  Nothing here allocates device memory; the one setting
// kept is the bound of the kernels' device-side waits (an atomic).
#include "libqad.h"

#include <math.h>

#include <atomic>
#include <mutex>

#include "qad_internal.h"

using qad::QuantizeArgs;

namespace {

// bound of the kernels' device-side waits, in microseconds (default 20 ms)
std::atomic<int64_t> g_wait_us{20000};

// Scratch of nvfp4_quantize_noalloc: the tensor records of the dynamic
// quantizer, in a fixed device array (every GPU the library runs on holds its
// own copy until the process ends).  Host code never uses the array's name
// as an address: its device address is taken per device with
// hipGetSymbolAddress, on the first call on that device with the device
// current, and kept.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// the current device's address of `scratch`, or nullptr on failure
void* static_scratch()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

} // namespace

namespace qad {
uint64_t wait_ticks() { return (uint64_t)g_wait_us.load(std::memory_order_relaxed) * 100u; }
} // namespace qad

namespace {

// 2^36 elements (128 GiB of bf16, 256 GiB of fp32: any tensor that fits in a
// GPU's memory) keeps byte offsets far from int64 overflow and every grid
// below 2^32 lanes
constexpr int64_t kMaxElems = (int64_t)1 << 36;

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }
inline int esize(qad_dtype_t t) { return t == QAD_BF16 ? 2 : 4; }
inline bool valid_dtype(qad_dtype_t t) { return t == QAD_F32 || t == QAD_BF16; }
inline hipStream_t hs(qad_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// B, R, C non-negative and B*R*C bounded; returns the element count or -1
int64_t tensor_elems(int64_t B, int64_t R, int64_t C)
{
    if (B < 0 || R < 0 || C < 0 || B > kMaxElems || R > kMaxElems || C > kMaxElems) return -1;
    if (B == 0 || R == 0 || C == 0) return 0;
    if (R > kMaxElems / C) return -1;
    const int64_t rc = R * C;
    if (B > kMaxElems / rc) return -1;
    return B * rc;
}

qad_status_t hip_status(hipError_t e) { return e == hipSuccess ? QAD_OK : QAD_ERR_HIP; }

// the per-tensor kernels launch B times the chunks of one tensor (the fp32
// chunks, the most numerous) workgroups in one grid; beyond 2^31 - 1 that
// grid cannot be expressed, so such a batch is a shape error
bool batch_grid_ok(int64_t B, int64_t rc)
{
    const int64_t P = qad::quantize_chunks(false, rc);
    return B <= 0 || P <= 0 || B <= (int64_t)0x7FFFFFFF / P;
}

uint32_t* ws_words(void* workspace) { return static_cast<uint32_t*>(workspace); }

// workspace of the tensor records for B tensors of rc elements (sized for
// fp32, whose 32 KiB chunks are the most numerous; bf16 needs less)
size_t record_bytes(int64_t B, int64_t rc)
{
    const int64_t P = qad::quantize_chunks(false, rc);
    return round256((size_t)B * (size_t)qad::record_words(P) * 4);
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

// fp8: per-tensor E4M3 (no block scales; frozen iff tscale_in is given;
// codes one byte per element, 8-byte aligned); otherwise NVFP4.
// static_ws: dynamic scales take their records from the library's fixed
// scratch (nvfp4_quantize_noalloc) instead of the caller's workspace, once
// every other argument has been checked.
qad_status_t quantize_impl(const void* x, qad_dtype_t xt, int64_t B, int64_t R, int64_t C,
                           const uint8_t* scales_in, const float* tscale_in, uint8_t* codes,
                           uint8_t* scales_out, float* tscale_out, void* y, void* workspace,
                           size_t ws_bytes, qad_stream_t stream, bool fp8 = false, bool static_ws = false)
{
    if (!valid_dtype(xt)) return QAD_ERR_DTYPE;
    const int64_t n = tensor_elems(B, R, C);
    if (n < 0 || C % (fp8 ? 8 : 16) != 0 || !batch_grid_ok(B, R * C)) return QAD_ERR_SHAPE;
    // frozen iff the tensor scales are given (the block scales of an empty
    // tensor may be NULL like every other empty buffer)
    if (!fp8 && scales_in && !tscale_in) return QAD_ERR_INVALID_ARG;
    const bool frozen = tscale_in != nullptr;
    if (n == 0) {
        // empty tensors: nothing to code; a tensor scale is still reported,
        // the frozen one as given and the dynamic one as for the zero tensor
        if (B == 0 || !tscale_out) return QAD_OK;
        if (!aligned(tscale_out, 4) || (tscale_in && !aligned(tscale_in, 4))) return QAD_ERR_ALIGNMENT;
        uint32_t* ts = reinterpret_cast<uint32_t*>(tscale_out);
        if (frozen)
            return hip_status(qad::launch_copy_u32(reinterpret_cast<const uint32_t*>(tscale_in), ts, B, hs(stream)));
        return hip_status(qad::launch_fill_u32(ts, B, 0x3F800000u, hs(stream)));   // 1.0f
    }
    if (!codes && !scales_out && !tscale_out && !y) return QAD_ERR_INVALID_ARG;
    if (!fp8 && frozen && !scales_in) return QAD_ERR_INVALID_ARG;
    if (!x) return QAD_ERR_INVALID_ARG;
    if (!aligned(x, 16) || (y && !aligned(y, 16)) || (codes && !aligned(codes, fp8 ? 8 : 4)) ||
        (tscale_in && !aligned(tscale_in, 4)) || (tscale_out && !aligned(tscale_out, 4)))
        return QAD_ERR_ALIGNMENT;
    const size_t xbytes = (size_t)n * esize(xt);
    if ((y && ranges_overlap(x, xbytes, y, (size_t)n * 2)) ||
        (codes && ranges_overlap(x, xbytes, codes, fp8 ? (size_t)n : (size_t)n / 2)) ||
        (scales_out && ranges_overlap(x, xbytes, scales_out, (size_t)n / 16)))
        return QAD_ERR_INVALID_ARG;
    if (!frozen && static_ws) {
        if (qad_workspace_bytes(QAD_OP_QUANTIZE, B, R, C) > kStaticScratchBytes) return QAD_ERR_WORKSPACE;
        workspace = static_scratch();
        if (!workspace) return QAD_ERR_HIP;
        ws_bytes = kStaticScratchBytes;
    }
    if (!frozen) {
        if (!workspace || ws_bytes < qad_workspace_bytes(QAD_OP_QUANTIZE, B, R, C)) return QAD_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return QAD_ERR_ALIGNMENT;
    }
    hipStream_t s = hs(stream);
    QuantizeArgs a;
    a.x = x;
    a.bf16 = xt == QAD_BF16;
    a.B = B;
    a.elems = R * C;
    a.scales_in = scales_in;
    a.tscale_in = tscale_in;
    a.codes = codes;
    a.scales_out = scales_out;
    a.tscale_out = tscale_out;
    a.y = static_cast<uint16_t*>(y);
    a.fp8 = fp8;
    a.wait_ticks = qad::wait_ticks();
    if (frozen) return hip_status(qad::launch_quantize(a, qad::QUANT_FROZEN, nullptr, s));
    // dynamic scales: one pass when every chunk of a tensor can be resident at
    // once, otherwise an amax pass first
    if (qad::quantize_one_pass_ok(a.bf16, fp8, B, a.elems))
        return hip_status(qad::launch_quantize(a, qad::QUANT_ONE_PASS, ws_words(workspace), s));
    hipError_t e = qad::launch_amax(x, a.bf16, B, a.elems, ws_words(workspace), s);
    if (e != hipSuccess) return QAD_ERR_HIP;
    return hip_status(qad::launch_quantize(a, qad::QUANT_AMAX_GIVEN, ws_words(workspace), s));
}

} // namespace

extern "C" {

const char* qad_status_string(qad_status_t status)
{
    switch (status) {
    case QAD_OK: return "QAD_OK";
    case QAD_ERR_INVALID_ARG: return "QAD_ERR_INVALID_ARG: invalid argument";
    case QAD_ERR_SHAPE: return "QAD_ERR_SHAPE: invalid shape";
    case QAD_ERR_DTYPE: return "QAD_ERR_DTYPE: unsupported dtype";
    case QAD_ERR_ALIGNMENT: return "QAD_ERR_ALIGNMENT: misaligned pointer";
    case QAD_ERR_WORKSPACE: return "QAD_ERR_WORKSPACE: workspace missing or too small";
    case QAD_ERR_NONFINITE: return "QAD_ERR_NONFINITE: non-finite value";
    case QAD_ERR_HIP: return "QAD_ERR_HIP: HIP runtime error";
    }
    return "unknown qad_status_t";
}

int qad_abi_version(void) { return 2; }

int64_t qad_set_wait_limit_us(int64_t us)
{
    if (us < 0) return g_wait_us.load(std::memory_order_relaxed);
    if (us > (int64_t)1 << 40) us = (int64_t)1 << 40;   // keeps the tick count far from overflow
    return g_wait_us.exchange(us, std::memory_order_relaxed);
}

size_t qad_workspace_bytes(qad_op_t op, int64_t B, int64_t R, int64_t C)
{
    // (B, R, C) of the W4A4 linear are (M, N, K): its operands are M x K and
    // N x K, each checked by the quantizer's own size; every other op takes a
    // batch of B tensors of R x C elements
    if (op == QAD_OP_W4A4_LINEAR) return round256(qad::linear_workspace_bytes(B, R, C));
    if (tensor_elems(B, R, C) < 0) return 0;
    switch (op) {
    case QAD_OP_AMAX:
    case QAD_OP_QUANTIZE:
    case QAD_OP_MSE_CALIBRATE: return record_bytes(B, R * C);
    case QAD_OP_KL: return round256(qad::kl_workspace_bytes(R, C));
    case QAD_OP_KL_TOPK:
    case QAD_OP_KL_TOPP: return round256(qad::kl_topk_workspace_bytes(R, C));
    case QAD_OP_W4A4_LINEAR: break;
    }
    return 0;
}

qad_status_t nvfp4_amax(const void* x, qad_dtype_t xt, int64_t B, int64_t R, int64_t C, float* amax_out,
                        void* workspace, size_t ws_bytes, qad_stream_t stream)
{
    if (!valid_dtype(xt)) return QAD_ERR_DTYPE;
    const int64_t n = tensor_elems(B, R, C);
    if (n < 0 || (C * esize(xt)) % 16 != 0 || !batch_grid_ok(B, R * C)) return QAD_ERR_SHAPE;
    if (B == 0) return QAD_OK;
    if (!amax_out) return QAD_ERR_INVALID_ARG;
    if (n > 0 && !x) return QAD_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(amax_out, 4)) return QAD_ERR_ALIGNMENT;
    hipStream_t s = hs(stream);
    uint32_t* out = reinterpret_cast<uint32_t*>(amax_out);
    if (n == 0) return hip_status(qad::launch_fill_u32(out, B, 0u, s));
    if (!workspace || ws_bytes < qad_workspace_bytes(QAD_OP_AMAX, B, R, C)) return QAD_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QAD_ERR_ALIGNMENT;
    hipError_t e = qad::launch_amax(x, xt == QAD_BF16, B, R * C, ws_words(workspace), s);
    if (e == hipSuccess) e = qad::launch_amax_out(ws_words(workspace), B, R * C, xt == QAD_BF16, out, s);
    return hip_status(e);
}

qad_status_t nvfp4_quantize(const void* x, qad_dtype_t xt, int64_t B, int64_t R, int64_t C,
                            const uint8_t* scales_in, const float* tscale_in, uint8_t* codes,
                            uint8_t* scales_out, float* tscale_out, void* y, void* workspace, size_t ws_bytes,
                            qad_stream_t stream)
{
    return quantize_impl(x, xt, B, R, C, scales_in, tscale_in, codes, scales_out, tscale_out, y, workspace,
                         ws_bytes, stream);
}

qad_status_t nvfp4_quantize_noalloc(const void* x, qad_dtype_t xt, int64_t B, int64_t R, int64_t C,
                                    const uint8_t* scales_in, const float* tscale_in, uint8_t* codes,
                                    uint8_t* scales_out, float* tscale_out, void* y, qad_stream_t stream)
{
    return quantize_impl(x, xt, B, R, C, scales_in, tscale_in, codes, scales_out, tscale_out, y, nullptr, 0, stream,
                         false, true);
}

qad_status_t nvfp4_qdq_fwd(const void* x, qad_dtype_t xt, int64_t B, int64_t R, int64_t C,
                           const uint8_t* scales_in, const float* tscale_in, void* y, void* workspace,
                           size_t ws_bytes, qad_stream_t stream)
{
    return quantize_impl(x, xt, B, R, C, scales_in, tscale_in, nullptr, nullptr, nullptr, y, workspace, ws_bytes,
                         stream);
}

qad_status_t fp8_quantize(const void* x, qad_dtype_t xt, int64_t B, int64_t R, int64_t C, const float* tscale_in,
                          uint8_t* codes, float* tscale_out, void* y, void* workspace, size_t ws_bytes,
                          qad_stream_t stream)
{
    return quantize_impl(x, xt, B, R, C, nullptr, tscale_in, codes, nullptr, tscale_out, y, workspace, ws_bytes,
                         stream, true);
}

qad_status_t nvfp4_qdq_bwd(const void* grad_y, void* grad_x, qad_dtype_t gt, int64_t n, qad_stream_t stream)
{
    if (!valid_dtype(gt)) return QAD_ERR_DTYPE;
    if (n < 0 || n > kMaxElems) return QAD_ERR_SHAPE;
    if (n == 0 || grad_x == grad_y) return QAD_OK;
    if (!grad_y || !grad_x) return QAD_ERR_INVALID_ARG;
    if (!aligned(grad_y, 16) || !aligned(grad_x, 16)) return QAD_ERR_ALIGNMENT;
    const size_t bytes = (size_t)n * esize(gt);
    if (ranges_overlap(grad_y, bytes, grad_x, bytes)) return QAD_ERR_INVALID_ARG;
    return hip_status(qad::launch_copy(grad_y, grad_x, (int64_t)bytes, hs(stream)));
}

qad_status_t nvfp4_qdq_bwd_clipped(const void* grad_y, qad_dtype_t gt, const void* x, qad_dtype_t xt,
                                   int64_t B, int64_t R, int64_t C, const uint8_t* scales,
                                   const float* tscale, void* grad_x, qad_stream_t stream)
{
    if (!valid_dtype(gt) || !valid_dtype(xt)) return QAD_ERR_DTYPE;
    const int64_t n = tensor_elems(B, R, C);
    if (n < 0 || C % 16 != 0) return QAD_ERR_SHAPE;
    if (n == 0) return QAD_OK;
    if (B > (int64_t)INT32_MAX / qad::clip_chunks(R * C)) return QAD_ERR_SHAPE;
    if (!grad_y || !x || !scales || !tscale || !grad_x) return QAD_ERR_INVALID_ARG;
    if (!aligned(grad_y, 16) || !aligned(x, 16) || !aligned(grad_x, 16) || !aligned(tscale, 4))
        return QAD_ERR_ALIGNMENT;
    const size_t gbytes = (size_t)n * esize(gt);
    if ((grad_x != grad_y && ranges_overlap(grad_y, gbytes, grad_x, gbytes)) ||
        ranges_overlap(x, (size_t)n * esize(xt), grad_x, gbytes) ||
        ranges_overlap(scales, (size_t)n / 16, grad_x, gbytes) ||
        ranges_overlap(tscale, (size_t)B * 4, grad_x, gbytes))
        return QAD_ERR_INVALID_ARG;
    qad::ClipArgs a;
    a.grad_y = grad_y;
    a.gbf16 = gt == QAD_BF16;
    a.x = x;
    a.xbf16 = xt == QAD_BF16;
    a.B = B;
    a.elems = R * C;
    a.scales = scales;
    a.tscale = tscale;
    a.grad_x = grad_x;
    return hip_status(qad::launch_qdq_bwd_clipped(a, hs(stream)));
}

qad_status_t nvfp4_frozen_sgd_step(const void* w, qad_dtype_t wt, const void* grad, qad_dtype_t gt,
                                   int64_t B, int64_t R, int64_t C, const uint8_t* scales,
                                   const float* tscale, float lr, float clip_coef, void* w_out,
                                   qad_stream_t stream)
{
    if (!valid_dtype(wt) || !valid_dtype(gt)) return QAD_ERR_DTYPE;
    const int64_t n = tensor_elems(B, R, C);
    if (n < 0 || C % 16 != 0) return QAD_ERR_SHAPE;
    if (!isfinite(lr) || !isfinite(clip_coef)) return QAD_ERR_INVALID_ARG;
    if (n == 0) return QAD_OK;
    if (B > (int64_t)INT32_MAX / qad::clip_chunks(R * C)) return QAD_ERR_SHAPE;
    if (!w || !grad || !scales || !tscale || !w_out) return QAD_ERR_INVALID_ARG;
    if (!aligned(w, 16) || !aligned(grad, 16) || !aligned(w_out, 16) || !aligned(tscale, 4))
        return QAD_ERR_ALIGNMENT;
    const size_t wbytes = (size_t)n * esize(wt);
    if ((w_out != w && ranges_overlap(w, wbytes, w_out, wbytes)) ||
        ranges_overlap(grad, (size_t)n * esize(gt), w_out, wbytes) ||
        ranges_overlap(scales, (size_t)n / 16, w_out, wbytes) ||
        ranges_overlap(tscale, (size_t)B * 4, w_out, wbytes))
        return QAD_ERR_INVALID_ARG;
    qad::SgdArgs a;
    a.w = w;
    a.wbf16 = wt == QAD_BF16;
    a.grad = grad;
    a.gbf16 = gt == QAD_BF16;
    a.B = B;
    a.elems = R * C;
    a.scales = scales;
    a.tscale = tscale;
    a.lr = lr;
    a.clip_coef = clip_coef;
    a.w_out = w_out;
    return hip_status(qad::launch_sgd_step(a, hs(stream)));
}

qad_status_t nvfp4_mse_calibrate(const void* w, qad_dtype_t wt, int64_t B, int64_t R, int64_t C,
                                 int32_t n_candidates, float k_min, float k_max, uint8_t* scales_out,
                                 float* tscale_out, void* workspace, size_t ws_bytes, qad_stream_t stream)
{
    if (!valid_dtype(wt)) return QAD_ERR_DTYPE;
    const int64_t n = tensor_elems(B, R, C);
    if (n < 0 || C % 16 != 0 || !batch_grid_ok(B, R * C)) return QAD_ERR_SHAPE;
    if (n_candidates < 1 || !(k_min > 0.0f) || !(k_max >= k_min) || !isfinite(k_max)) return QAD_ERR_INVALID_ARG;
    // consecutive candidates must not be able to skip an E4M3 value (relative
    // step at most 1/16, below the narrowest E4M3 rounding interval, 1/15)
    if (n_candidates > 1 && ((double)k_max - (double)k_min) / (double)(n_candidates - 1) > (double)k_min / 16.0)
        return QAD_ERR_INVALID_ARG;
    if (n == 0) {
        // empty tensors: no block scales; the tensor scale of the zero tensor
        if (B == 0 || !tscale_out) return QAD_OK;
        if (!aligned(tscale_out, 4)) return QAD_ERR_ALIGNMENT;
        return hip_status(qad::launch_fill_u32(reinterpret_cast<uint32_t*>(tscale_out), B, 0x3F800000u, hs(stream)));
    }
    if (!w || !scales_out || !tscale_out) return QAD_ERR_INVALID_ARG;
    if (!aligned(w, 16) || !aligned(tscale_out, 4)) return QAD_ERR_ALIGNMENT;
    if (!workspace || ws_bytes < qad_workspace_bytes(QAD_OP_MSE_CALIBRATE, B, R, C)) return QAD_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QAD_ERR_ALIGNMENT;
    hipStream_t s = hs(stream);
    qad::MseArgs a;
    a.w = w;
    a.bf16 = wt == QAD_BF16;
    a.B = B;
    a.elems = R * C;
    a.k_lo = k_min;
    a.k_hi = n_candidates > 1 ? k_max : k_min;
    a.scales_out = scales_out;
    a.tscale_out = tscale_out;
    return hip_status(qad::launch_mse_calibrate(a, ws_words(workspace), s));
}

qad_status_t qad_kl_fwd_bwd(const void* teacher, const void* student, qad_dtype_t lt, int64_t tokens,
                            int64_t vocab, float temperature, float grad_scale, float* loss_out,
                            float* row_loss, void* grad_student, qad_dtype_t gt, void* workspace,
                            size_t ws_bytes, qad_stream_t stream)
{
    if (!valid_dtype(lt) || (grad_student && !valid_dtype(gt))) return QAD_ERR_DTYPE;
    const int64_t n = tensor_elems(1, tokens, vocab);
    if (n < 0 || vocab % 8 != 0 || tokens > 0x7FFFFFFFll) return QAD_ERR_SHAPE;
    if (!(temperature > 0.0f) || !isfinite(temperature) || !isfinite(grad_scale)) return QAD_ERR_INVALID_ARG;
    if (!loss_out) return QAD_ERR_INVALID_ARG;
    if (tokens > 0 && vocab == 0) return QAD_ERR_SHAPE;
    if (n > 0 && (!teacher || !student)) return QAD_ERR_INVALID_ARG;
    if (!aligned(teacher, 16) || !aligned(student, 16) || (grad_student && !aligned(grad_student, 16)) ||
        !aligned(loss_out, 4) || (row_loss && !aligned(row_loss, 4)))
        return QAD_ERR_ALIGNMENT;
    if (grad_student) {
        const size_t ib = (size_t)n * esize(lt), gb = (size_t)n * esize(gt);
        if (ranges_overlap(teacher, ib, grad_student, gb) || ranges_overlap(student, ib, grad_student, gb))
            return QAD_ERR_INVALID_ARG;
    }
    if (tokens > 0) {
        if (!workspace || ws_bytes < qad_workspace_bytes(QAD_OP_KL, 1, tokens, vocab)) return QAD_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return QAD_ERR_ALIGNMENT;
    }
    float* rows = row_loss ? row_loss : static_cast<float*>(workspace);
    qad::KlArgs a;
    a.teacher = teacher;
    a.student = student;
    a.bf16_in = lt == QAD_BF16;
    a.tokens = tokens;
    a.vocab = vocab;
    a.temperature = temperature;
    a.grad_scale = grad_scale;
    a.row_loss = rows;
    a.loss_out = loss_out;
    a.grad = grad_student;
    a.grad_bf16 = gt == QAD_BF16;
    a.wait_ticks = qad::wait_ticks();
    return hip_status(qad::launch_kl(a, workspace, hs(stream)));
}

qad_status_t qad_kl_topk_fwd_bwd(const void* teacher, const void* student, qad_dtype_t lt, int64_t tokens,
                                 int64_t vocab, int64_t k, float temperature, float grad_scale, float* loss_out,
                                 float* row_loss, void* grad_student, qad_dtype_t gt, void* workspace,
                                 size_t ws_bytes, qad_stream_t stream)
{
    if (!valid_dtype(lt) || (grad_student && !valid_dtype(gt))) return QAD_ERR_DTYPE;
    const int64_t n = tensor_elems(1, tokens, vocab);
    if (n < 0 || vocab % 8 != 0 || tokens > 0x7FFFFFFFll || vocab > 0x7FFFFFFFll) return QAD_ERR_SHAPE;
    if (tokens > 0 && vocab == 0) return QAD_ERR_SHAPE;
    if (k < 1) return QAD_ERR_INVALID_ARG;
    if (!(temperature > 0.0f) || !isfinite(temperature) || !isfinite(grad_scale)) return QAD_ERR_INVALID_ARG;
    if (!loss_out) return QAD_ERR_INVALID_ARG;
    if (n > 0 && (!teacher || !student)) return QAD_ERR_INVALID_ARG;
    if (!aligned(teacher, 16) || !aligned(student, 16) || (grad_student && !aligned(grad_student, 16)) ||
        !aligned(loss_out, 4) || (row_loss && !aligned(row_loss, 4)))
        return QAD_ERR_ALIGNMENT;
    if (grad_student) {
        const size_t ib = (size_t)n * esize(lt), gb = (size_t)n * esize(gt);
        if (ranges_overlap(teacher, ib, grad_student, gb) || ranges_overlap(student, ib, grad_student, gb))
            return QAD_ERR_INVALID_ARG;
    }
    if (tokens > 0) {
        if (!workspace || ws_bytes < qad_workspace_bytes(QAD_OP_KL_TOPK, 1, tokens, vocab)) return QAD_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return QAD_ERR_ALIGNMENT;
    }
    qad::KlArgs a;
    a.teacher = teacher;
    a.student = student;
    a.bf16_in = lt == QAD_BF16;
    a.tokens = tokens;
    a.vocab = vocab;
    a.temperature = temperature;
    a.grad_scale = grad_scale;
    a.row_loss = row_loss ? row_loss : static_cast<float*>(workspace);
    a.loss_out = loss_out;
    a.grad = grad_student;
    a.grad_bf16 = gt == QAD_BF16;
    a.wait_ticks = qad::wait_ticks();
    return hip_status(qad::launch_kl_topk(a, k, workspace, hs(stream)));
}

qad_status_t qad_kl_topp_fwd_bwd(const void* teacher, const void* student, qad_dtype_t lt, int64_t tokens,
                                 int64_t vocab, float top_p, float temperature, float grad_scale, float* loss_out,
                                 float* row_loss, void* grad_student, qad_dtype_t gt, float* tau_out,
                                 void* workspace, size_t ws_bytes, qad_stream_t stream)
{
    if (!valid_dtype(lt) || (grad_student && !valid_dtype(gt))) return QAD_ERR_DTYPE;
    const int64_t n = tensor_elems(1, tokens, vocab);
    if (n < 0 || vocab % 8 != 0 || tokens > 0x7FFFFFFFll || vocab > 0x7FFFFFFFll) return QAD_ERR_SHAPE;
    if (tokens > 0 && vocab == 0) return QAD_ERR_SHAPE;
    if (!(top_p > 0.0f) || !isfinite(top_p)) return QAD_ERR_INVALID_ARG;
    if (!(temperature > 0.0f) || !isfinite(temperature) || !isfinite(grad_scale)) return QAD_ERR_INVALID_ARG;
    if (!loss_out) return QAD_ERR_INVALID_ARG;
    if (n > 0 && (!teacher || !student)) return QAD_ERR_INVALID_ARG;
    if (!aligned(teacher, 16) || !aligned(student, 16) || (grad_student && !aligned(grad_student, 16)) ||
        !aligned(loss_out, 4) || (row_loss && !aligned(row_loss, 4)) || (tau_out && !aligned(tau_out, 4)))
        return QAD_ERR_ALIGNMENT;
    const size_t ib = (size_t)n * esize(lt), gb = grad_student ? (size_t)n * esize(gt) : 0;
    if (grad_student && (ranges_overlap(teacher, ib, grad_student, gb) || ranges_overlap(student, ib, grad_student, gb)))
        return QAD_ERR_INVALID_ARG;
    if (tau_out && tokens > 0) {
        const size_t tb = (size_t)tokens * 4;
        if (ranges_overlap(tau_out, tb, teacher, ib) || ranges_overlap(tau_out, tb, student, ib) ||
            (grad_student && ranges_overlap(tau_out, tb, grad_student, gb)) ||
            ranges_overlap(tau_out, tb, loss_out, 4) || (row_loss && ranges_overlap(tau_out, tb, row_loss, tb)))
            return QAD_ERR_INVALID_ARG;
    }
    if (tokens > 0) {
        if (!workspace || ws_bytes < qad_workspace_bytes(QAD_OP_KL_TOPP, 1, tokens, vocab)) return QAD_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return QAD_ERR_ALIGNMENT;
        if (tau_out && ranges_overlap(tau_out, (size_t)tokens * 4, workspace, ws_bytes)) return QAD_ERR_INVALID_ARG;
    }
    qad::KlArgs a;
    a.teacher = teacher;
    a.student = student;
    a.bf16_in = lt == QAD_BF16;
    a.tokens = tokens;
    a.vocab = vocab;
    a.temperature = temperature;
    a.grad_scale = grad_scale;
    a.row_loss = row_loss ? row_loss : static_cast<float*>(workspace);
    a.loss_out = loss_out;
    a.grad = grad_student;
    a.grad_bf16 = gt == QAD_BF16;
    a.wait_ticks = qad::wait_ticks();
    return hip_status(qad::launch_kl_topp(a, top_p, tau_out, workspace, hs(stream)));
}

qad_status_t qad_check_finite(const float* values, int64_t n, qad_stream_t stream)
{
    if (n < 0) return QAD_ERR_SHAPE;
    if (n == 0) return QAD_OK;
    if (!values) return QAD_ERR_INVALID_ARG;
    if (hipStreamSynchronize(hs(stream)) != hipSuccess) return QAD_ERR_HIP;
    float buf[256];
    for (int64_t off = 0; off < n; off += 256) {
        const int64_t k = n - off < 256 ? n - off : 256;
        if (hipMemcpy(buf, values + off, (size_t)k * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
            return QAD_ERR_HIP;
        for (int64_t i = 0; i < k; ++i)
            if (!isfinite(buf[i])) return QAD_ERR_NONFINITE;
    }
    return QAD_OK;
}

} // extern "C"
