// Internal launch interface between the C-ABI layer (libqad.hip) and the
// kernel files.  Every launcher enqueues on `stream` and returns the HIP
// error of its launches; all shapes were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qad {

// out[i] = v for i < n (graph-safe replacement for a memset)
hipError_t launch_fill_u32(uint32_t* out, int64_t n, uint32_t v, hipStream_t stream);
// n words from src to dst (4-byte aligned, no overlap)
hipError_t launch_copy_u32(const uint32_t* src, uint32_t* dst, int64_t n, hipStream_t stream);

// Words of one tensor's record in the workspace for a tensor cut into P
// chunks (amax publication, sub-group counters, broadcast slots).
__host__ __device__ inline int64_t record_words(int64_t P)
{
    const int64_t w = 32 + 32 * ((P + 15) / 16) + 16 * P;
    return (w + 31) & ~(int64_t)31;
}
// chunks (32 KiB of input) per tensor of `elems` elements
int64_t quantize_chunks(bool bf16, int64_t elems);
int64_t amax_chunks(int64_t bytes_per_tensor);

// Tensor amax of B tensors of `elems` elements (elems * esize % 16 == 0) into
// the tensor records at ws (zeroes them first); word 0 of record b ends as
// the amax of tensor b (binary32 bits).
hipError_t launch_amax(const void* x, bool bf16, int64_t B, int64_t elems, uint32_t* ws, hipStream_t stream);
// copy the amax of every record to out[B]
hipError_t launch_amax_out(const uint32_t* ws, int64_t B, int64_t elems, bool bf16, uint32_t* out,
                           hipStream_t stream);

struct QuantizeArgs {
    const void* x;
    bool bf16;
    int64_t B;
    int64_t elems;             // R * C per tensor, multiple of 16 (NVFP4) or 8 (FP8)
    const uint8_t* scales_in;  // frozen block scales or null (dynamic)
    const float* tscale_in;    // frozen tensor scales
    uint8_t* codes;
    uint8_t* scales_out;
    float* tscale_out;
    uint16_t* y;
    bool fp8 = false;          // FP8 (E4M3) per-tensor QDQ: no block scales, codes one byte per element
    uint64_t wait_ticks = 0;   // bound of the one-pass amax wait (100 MHz ticks), from wait_ticks()
};
enum { QUANT_FROZEN = 0, QUANT_AMAX_GIVEN = 1, QUANT_ONE_PASS = 2 };
// whether every chunk of one tensor can be resident at once with room to spare
bool quantize_one_pass_ok(bool bf16, bool fp8, int64_t B, int64_t elems);
// QUANT_AMAX_GIVEN expects launch_amax's records in ws; QUANT_ONE_PASS
// zeroes and uses them itself; QUANT_FROZEN ignores ws.
hipError_t launch_quantize(const QuantizeArgs& a, int mode, uint32_t* ws, hipStream_t stream);

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

struct ClipArgs {
    const void* grad_y;
    bool gbf16;
    const void* x;             // the forward's input
    bool xbf16;
    int64_t B;
    int64_t elems;             // R * C per tensor, multiple of 16
    const uint8_t* scales;     // [B][elems/16] block scale codes the forward used
    const float* tscale;       // [B] tensor scales the forward used
    void* grad_x;              // dtype of grad_y
};
// workgroups per tensor of the clipped backward
int64_t clip_chunks(int64_t elems);
hipError_t launch_qdq_bwd_clipped(const ClipArgs& a, hipStream_t stream);

struct SgdArgs {
    const void* w;             // weights before the step (the forward's input)
    bool wbf16;
    const void* grad;          // gradient wrt the QDQ output
    bool gbf16;
    int64_t B;
    int64_t elems;             // R * C per tensor, multiple of 16
    const uint8_t* scales;     // [B][elems/16] frozen block scale codes
    const float* tscale;       // [B] frozen tensor scales
    float lr;
    float clip_coef;
    void* w_out;               // dtype of w; may be w
};
// frozen-scale SGD step: launch shape of the clipped backward
hipError_t launch_sgd_step(const SgdArgs& a, hipStream_t stream);

struct MseArgs {
    const void* w;
    bool bf16;
    int64_t B;
    int64_t elems;
    float k_lo, k_hi;          // first and last candidate multipliers
    uint8_t* scales_out;
    float* tscale_out;
};
// amax records in ws, then the search
hipError_t launch_mse_calibrate(const MseArgs& a, uint32_t* ws, hipStream_t stream);

struct KlArgs {
    const void* teacher;
    const void* student;
    bool bf16_in;
    int64_t tokens, vocab;
    float temperature, grad_scale;
    float* row_loss;           // [tokens], never null (start of the workspace if the caller has none)
    float* loss_out;
    void* grad;                // null: forward only
    bool grad_bf16;
    const float* tau = nullptr;  // teacher-top-k thresholds per row (null: full vocabulary)
    uint64_t wait_ticks = 0;     // bound of the segment kernels' row exchange wait (100 MHz ticks)
    float inv_t = 1.0f;          // 1 / temperature (set by the launchers)
    float lgmul = 0.0f;          // log2 |grad_scale / temperature| (set by the launchers)
};
// the process-wide bound of the kernels' device-side waits, in ticks of the
// 100 MHz wall clock (qad_set_wait_limit_us)
uint64_t wait_ticks();
// scratch of launch_kl: per-row losses, then per-row exchange records
size_t kl_workspace_bytes(int64_t tokens, int64_t vocab);
hipError_t launch_kl(const KlArgs& a, void* workspace, hipStream_t stream);
// teacher-top-k KL (k >= 1): the KL workspace followed by per-row thresholds
size_t kl_topk_workspace_bytes(int64_t tokens, int64_t vocab);
hipError_t launch_kl_topk(const KlArgs& a, int64_t k, void* workspace, hipStream_t stream);
// teacher-top-p (nucleus) KL; thresholds into tau_out when non-null, else into
// the workspace slot of the top-k layout (kl_topk_workspace_bytes)
hipError_t launch_kl_topp(const KlArgs& a, float top_p, float* tau_out, void* workspace, hipStream_t stream);

// W4A4 linear: the QDQ records of the larger operand, then the GEMM scratch
size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K);

} // namespace qad
