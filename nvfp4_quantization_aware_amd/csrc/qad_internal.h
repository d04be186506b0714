// Internal launch interface between the C-ABI layer (libqad.hip) and the
// kernel files.  Every launcher enqueues on `stream` and returns the HIP
// error of its launches; all shapes were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qad {

constexpr int kThreads = 256;

// out[i] = v for i < n (graph-safe replacement for a memset)
hipError_t launch_fill_u32(uint32_t* out, int64_t n, uint32_t v, hipStream_t stream);

// amax of B tensors of `elems` elements (elems * esize % 16 == 0); result as
// binary32 bit patterns, max-accumulated into amax_bits[B] (which must be
// zero or a lower bound beforehand).
hipError_t launch_amax(const void* x, bool bf16, int64_t B, int64_t elems, uint32_t* amax_bits,
                       hipStream_t stream);

struct QuantizeArgs {
    const void* x;
    bool bf16;
    int64_t B;
    int64_t elems;             // R * C per tensor, multiple of 16
    const uint8_t* scales_in;  // frozen block scales or null (dynamic)
    const float* tscale_in;    // frozen tensor scales
    const uint32_t* amax_bits; // dynamic: per-tensor amax from launch_amax
    uint8_t* codes;
    uint8_t* scales_out;
    float* tscale_out;
    uint16_t* y;
};
hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t stream);

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

struct MseArgs {
    const void* w;
    bool bf16;
    int64_t B;
    int64_t elems;
    float k_lo, k_hi;          // first and last candidate multipliers
    const uint32_t* amax_bits;
    uint8_t* scales_out;
    float* tscale_out;
};
hipError_t launch_mse_calibrate(const MseArgs& a, hipStream_t stream);

struct KlArgs {
    const void* teacher;
    const void* student;
    bool bf16_in;
    int64_t tokens, vocab;
    float temperature, grad_scale;
    float* row_loss;           // [tokens], never null (workspace if needed)
    float* loss_out;
    void* grad;                // null: forward only
    bool grad_bf16;
};
hipError_t launch_kl(const KlArgs& a, hipStream_t stream);

} // namespace qad
