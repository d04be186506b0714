// NVFP4 simulated-quantization kernels for gfx950: tensor amax, quantize /
// dequantize with dynamic or frozen scales, the straight-through copy and the
// MSE block-scale search.  Page legend and numerical conventions: see
// include/libqad.h.  All kernels are HBM-streaming (no MFMA: nothing here is a
// contraction); 16-byte loads and stores, one wave-lane pair per 16-element
// block for the quantizer.
#include "qad_device.h"
#include "qad_internal.h"

namespace qad {
namespace {

// RN(1/6) in binary32 (0x3E2AAAAB)
constexpr float kRcp6 = 0x1.555556p-3f;
// Tensor scales at or above this use the reciprocal division (its validity
// range); smaller ones take IEEE division everywhere.
constexpr float kFastMinScale = 0x1p-80f;
// Units of 8 elements handled per lane per tile of the quantizer.
constexpr int kUnroll = 4;
// Workgroups to aim for per launch (16 per compute unit on 256 CUs).
constexpr int64_t kTargetGroups = 4096;

__global__ void fill_u32_kernel(uint32_t* out, int64_t n, uint32_t v)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) out[i] = v;
}

// ---------------------------------------------------------------------------
// Tensor amax ([Lightning] "量化尺度处理策略": dynamic scales start from the
// max of each tensor, recomputed every step).  The magnitude of a finite
// binary32 / bf16 value orders like its bit pattern with the sign cleared, so
// the maximum is an integer max: exact and independent of evaluation order.
// One atomicMax per workgroup per tensor.
// ---------------------------------------------------------------------------
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

template <bool BF16>
__device__ __forceinline__ uint32_t absmax_vec(const uint4& v, uint32_t m)
{
    if constexpr (BF16) {
        us2 acc = __builtin_bit_cast(us2, m);
        acc = __builtin_elementwise_max(acc, __builtin_bit_cast(us2, v.x & 0x7FFF7FFFu));
        acc = __builtin_elementwise_max(acc, __builtin_bit_cast(us2, v.y & 0x7FFF7FFFu));
        acc = __builtin_elementwise_max(acc, __builtin_bit_cast(us2, v.z & 0x7FFF7FFFu));
        acc = __builtin_elementwise_max(acc, __builtin_bit_cast(us2, v.w & 0x7FFF7FFFu));
        return __builtin_bit_cast(uint32_t, acc);
    } else {
        m = umax(m, v.x & 0x7FFFFFFFu);
        m = umax(m, v.y & 0x7FFFFFFFu);
        m = umax(m, v.z & 0x7FFFFFFFu);
        m = umax(m, v.w & 0x7FFFFFFFu);
        return m;
    }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void amax_kernel(const uint4* __restrict__ x, int64_t vecs, int groups,
                                                        uint32_t* __restrict__ amax_bits)
{
    const int b = blockIdx.x / groups, g = blockIdx.x - b * groups;
    const uint4* xb = x + (int64_t)b * vecs;
    const int64_t stride = (int64_t)groups * kThreads;
    int64_t i = (int64_t)g * kThreads + threadIdx.x;
    uint32_t m = 0;
    for (; i + 3 * stride < vecs; i += 4 * stride) {
        const uint4 v0 = xb[i], v1 = xb[i + stride], v2 = xb[i + 2 * stride], v3 = xb[i + 3 * stride];
        m = absmax_vec<BF16>(v0, m);
        m = absmax_vec<BF16>(v1, m);
        m = absmax_vec<BF16>(v2, m);
        m = absmax_vec<BF16>(v3, m);
    }
    for (; i < vecs; i += stride) m = absmax_vec<BF16>(xb[i], m);
    if constexpr (BF16) m = umax(m & 0xFFFFu, m >> 16) << 16; // bf16 bits -> binary32 bits
    m = wave_max_u32(m);
    __shared__ uint32_t part[kThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kThreads / 64; ++w) m = umax(m, part[w]);
        if (m) atomicMax(amax_bits + b, m);
    }
}

// ---------------------------------------------------------------------------
// Per-tensor tables in LDS: effective scale dec(c) * s_g of every E4M3 code c
// and its correctly rounded reciprocal (0 for a zero scale).
// ---------------------------------------------------------------------------
struct ScaleTable {
    float seff[128];
    float rcp[128];
};

__device__ __forceinline__ void build_table(ScaleTable& tab, float s_g)
{
    const int t = threadIdx.x;
    if (t < 128) {
        const float se = e4m3_decode((uint32_t)t) * s_g;
        tab.seff[t] = se;
        tab.rcp[t] = se > 0.0f ? 1.0f / se : 0.0f;
    }
}

// Block scale code from a block amax ([Nano]: E4M3 scale per block):
// E4M3((amax_b / 6) / s_g), both quotients correctly rounded.
template <bool FAST>
__device__ __forceinline__ uint32_t block_scale_code(float amax_b, float s_g, float rcp_g)
{
    float t1, raw;
    if constexpr (FAST) {
        t1 = div_rcp(amax_b, 6.0f, kRcp6);
        raw = div_rcp(t1, s_g, rcp_g);
    } else {
        t1 = amax_b / 6.0f;
        raw = t1 / s_g;
    }
    return e4m3_encode(raw);
}

// E2M1 magnitude index of x / s (s = 0 gives index 0)
template <bool FAST>
__device__ __forceinline__ uint32_t element_index(float x, float s, float r)
{
    float q;
    if constexpr (FAST) q = div_rcp(x, s, r);
    else q = s > 0.0f ? x / s : 0.0f;
    return e2m1_index(q);
}

template <bool BF16>
__device__ __forceinline__ void load_unit(const void* x, int64_t unit, bool valid, float (&e)[8])
{
    if constexpr (BF16) {
        uint4 v = valid ? reinterpret_cast<const uint4*>(x)[unit] : make_uint4(0, 0, 0, 0);
        e[0] = bf_lo(v.x); e[1] = bf_hi(v.x); e[2] = bf_lo(v.y); e[3] = bf_hi(v.y);
        e[4] = bf_lo(v.z); e[5] = bf_hi(v.z); e[6] = bf_lo(v.w); e[7] = bf_hi(v.w);
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(x) + 2 * unit;
        uint4 v0 = valid ? p[0] : make_uint4(0, 0, 0, 0);
        uint4 v1 = valid ? p[1] : make_uint4(0, 0, 0, 0);
        e[0] = as_f(v0.x); e[1] = as_f(v0.y); e[2] = as_f(v0.z); e[3] = as_f(v0.w);
        e[4] = as_f(v1.x); e[5] = as_f(v1.y); e[6] = as_f(v1.z); e[7] = as_f(v1.w);
    }
}

// ---------------------------------------------------------------------------
// Quantize / dequantize.  A lane owns a "unit" of 8 consecutive elements; the
// lane pair (2k, 2k+1) owns one 16-element block and exchanges its half-block
// amax through DPP.  Per element: code = E2M1(x / s_eff) (sign from x),
// y = bf16(dec(code) * s_eff).
// ---------------------------------------------------------------------------
template <bool BF16, bool FROZEN, bool FAST>
__device__ __forceinline__ void quantize_tensor(const QuantizeArgs& a, int b, int g, int groups,
                                                const ScaleTable& tab, float s_g)
{
    const int64_t units = a.elems >> 3;
    const int64_t ubase = (int64_t)b * units;
    const float rcp_g = 1.0f / s_g;
    constexpr int64_t kTile = (int64_t)kThreads * kUnroll;
    const int t = threadIdx.x;
    for (int64_t tile = g; tile * kTile < units; tile += groups) {
        float e[kUnroll][8];
        bool valid[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t u = tile * kTile + k * kThreads + t;
            valid[k] = u < units;
            load_unit<BF16>(a.x, ubase + u, valid[k], e[k]);
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t u = tile * kTile + k * kThreads + t;
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) m = umax(m, as_u(e[k][i]) & 0x7FFFFFFFu);
            m = umax(m, swap_pair(m));
            uint32_t sb;
            if constexpr (FROZEN) sb = valid[k] ? a.scales_in[(ubase + u) >> 1] : 0u;
            else sb = block_scale_code<FAST>(as_f(m), s_g, rcp_g);
            sb &= 127u;
            const float s = tab.seff[sb], r = tab.rcp[sb];
            uint32_t code = 0, yw[4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const uint32_t i0 = element_index<FAST>(e[k][i], s, r);
                const uint32_t i1 = element_index<FAST>(e[k][i + 1], s, r);
                code |= (i0 | ((as_u(e[k][i]) >> 31) << 3)) << (4 * i);
                code |= (i1 | ((as_u(e[k][i + 1]) >> 31) << 3)) << (4 * i + 4);
                const float y0 = __builtin_copysignf(e2m1_value(i0) * s, e[k][i]);
                const float y1 = __builtin_copysignf(e2m1_value(i1) * s, e[k][i + 1]);
                yw[i >> 1] = pack_bf16x2(y0, y1);
            }
            if (valid[k]) {
                if (a.y) reinterpret_cast<uint4*>(a.y)[ubase + u] = make_uint4(yw[0], yw[1], yw[2], yw[3]);
                if (a.codes) reinterpret_cast<uint32_t*>(a.codes)[ubase + u] = code;
                if (a.scales_out && !(t & 1)) a.scales_out[(ubase + u) >> 1] = (uint8_t)sb;
            }
        }
    }
}

template <bool BF16, bool FROZEN>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantizeArgs a, int groups)
{
    __shared__ ScaleTable tab;
    const int b = blockIdx.x / groups, g = blockIdx.x - b * groups;
    float s_g;
    if constexpr (FROZEN) {
        s_g = a.tscale_in[b];
    } else {
        const float amax = as_f(a.amax_bits[b]);
        s_g = amax > 0.0f ? amax / 2688.0f : 1.0f;
    }
    build_table(tab, s_g);
    if (g == 0 && threadIdx.x == 0 && a.tscale_out) a.tscale_out[b] = s_g;
    __syncthreads();
    if (s_g >= kFastMinScale) quantize_tensor<BF16, FROZEN, true>(a, b, g, groups, tab, s_g);
    else quantize_tensor<BF16, FROZEN, false>(a, b, g, groups, tab, s_g);
}

// ---------------------------------------------------------------------------
// Straight-through backward: a 16-byte vector copy.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        int64_t vecs, const uint16_t* __restrict__ src_tail,
                                                        uint16_t* __restrict__ dst_tail, int tail_halves)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + 3 * stride < vecs; i += 4 * stride) {
        const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
        dst[i] = v0;
        dst[i + stride] = v1;
        dst[i + 2 * stride] = v2;
        dst[i + 3 * stride] = v3;
    }
    for (; i < vecs; i += stride) dst[i] = src[i];
    if (blockIdx.x == 0 && threadIdx.x < tail_halves) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}

// ---------------------------------------------------------------------------
// MSE calibration of the frozen block scales ([Lightning] "量化尺度处理策略").
// One lane per 16-element block.  The candidates amax_b * k_i / 6 rounded to
// E4M3 are non-decreasing in i and, for grids no coarser than k_min/16 per
// step, visit every code between the first and the last candidate's code
// without a gap.  So the search runs over that contiguous code range (at most
// 9 codes for k in [0.5, 1]) instead of all n candidates; ascending order
// keeps "first candidate with strictly smaller error" as the tie rule.
// ---------------------------------------------------------------------------
template <bool FAST>
__device__ __forceinline__ float block_error(const float (&e)[16], float s, float r)
{
    float err = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t idx = element_index<FAST>(e[j], s, r);
        const float d = __builtin_fabsf(e[j]) - e2m1_value(idx) * s;
        err = err + d * d;
    }
    return err;
}

template <bool BF16, bool FAST>
__device__ __forceinline__ void calibrate_tensor(const MseArgs& a, int b, int g, int groups,
                                                 const ScaleTable& tab, float s_g)
{
    const int64_t nblk = a.elems >> 4;
    const float rcp_g = 1.0f / s_g;
    const int64_t stride = (int64_t)groups * kThreads;
    for (int64_t blk = (int64_t)g * kThreads + threadIdx.x; blk < nblk; blk += stride) {
        const int64_t gb = (int64_t)b * nblk + blk;
        float e[16];
        if constexpr (BF16) {
            const uint4* p = reinterpret_cast<const uint4*>(a.w) + 2 * gb;
            const uint4 v0 = p[0], v1 = p[1];
            const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) { e[2 * j] = bf_lo(w[j]); e[2 * j + 1] = bf_hi(w[j]); }
        } else {
            const uint4* p = reinterpret_cast<const uint4*>(a.w) + 4 * gb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 v = p[j];
                e[4 * j] = as_f(v.x); e[4 * j + 1] = as_f(v.y); e[4 * j + 2] = as_f(v.z); e[4 * j + 3] = as_f(v.w);
            }
        }
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) m = umax(m, as_u(e[j]) & 0x7FFFFFFFu);
        const float amax_b = as_f(m);
        const uint32_t c_lo = block_scale_code<FAST>(amax_b * a.k_lo, s_g, rcp_g);
        const uint32_t c_hi = block_scale_code<FAST>(amax_b * a.k_hi, s_g, rcp_g);
        uint32_t best = c_lo;
        float best_err = __builtin_inff();
        for (uint32_t c = c_lo; c <= c_hi; ++c) {
            const float err = block_error<FAST>(e, tab.seff[c], tab.rcp[c]);
            if (err < best_err) { best_err = err; best = c; }
        }
        a.scales_out[gb] = (uint8_t)best;
    }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void mse_kernel(MseArgs a, int groups)
{
    __shared__ ScaleTable tab;
    const int b = blockIdx.x / groups, g = blockIdx.x - b * groups;
    const float amax = as_f(a.amax_bits[b]);
    const float s_g = amax > 0.0f ? amax / 2688.0f : 1.0f;
    build_table(tab, s_g);
    if (g == 0 && threadIdx.x == 0) a.tscale_out[b] = s_g;
    __syncthreads();
    if (s_g >= kFastMinScale) calibrate_tensor<BF16, true>(a, b, g, groups, tab, s_g);
    else calibrate_tensor<BF16, false>(a, b, g, groups, tab, s_g);
}

int groups_for(int64_t B, int64_t work_items, int64_t per_group)
{
    int64_t need = (work_items + per_group - 1) / per_group;
    int64_t want = (kTargetGroups + B - 1) / B;
    int64_t g = need < want ? need : want;
    if (g < 1) g = 1;
    if (g * B > 0x7FFFFFFFll) g = 0x7FFFFFFFll / B;
    return (int)g;
}

} // namespace

hipError_t launch_fill_u32(uint32_t* out, int64_t n, uint32_t v, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    int64_t grid = (n + kThreads - 1) / kThreads;
    if (grid > 1024) grid = 1024;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, out, n, v);
    return hipGetLastError();
}

hipError_t launch_amax(const void* x, bool bf16, int64_t B, int64_t elems, uint32_t* amax_bits, hipStream_t stream)
{
    const int64_t vecs = elems * (bf16 ? 2 : 4) / 16;
    if (B <= 0 || vecs <= 0) return hipSuccess;
    const int groups = groups_for(B, vecs, (int64_t)kThreads * 16);
    const dim3 grid((unsigned)(groups * B));
    if (bf16) hipLaunchKernelGGL(amax_kernel<true>, grid, dim3(kThreads), 0, stream,
                                 (const uint4*)x, vecs, groups, amax_bits);
    else hipLaunchKernelGGL(amax_kernel<false>, grid, dim3(kThreads), 0, stream,
                            (const uint4*)x, vecs, groups, amax_bits);
    return hipGetLastError();
}

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t stream)
{
    if (a.B <= 0 || a.elems <= 0) return hipSuccess;
    const int groups = groups_for(a.B, a.elems >> 3, (int64_t)kThreads * kUnroll);
    const dim3 grid((unsigned)(groups * a.B));
    const bool frozen = a.scales_in != nullptr;
    if (a.bf16 && frozen) hipLaunchKernelGGL((quantize_kernel<true, true>), grid, dim3(kThreads), 0, stream, a, groups);
    else if (a.bf16) hipLaunchKernelGGL((quantize_kernel<true, false>), grid, dim3(kThreads), 0, stream, a, groups);
    else if (frozen) hipLaunchKernelGGL((quantize_kernel<false, true>), grid, dim3(kThreads), 0, stream, a, groups);
    else hipLaunchKernelGGL((quantize_kernel<false, false>), grid, dim3(kThreads), 0, stream, a, groups);
    return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream)
{
    const int64_t vecs = bytes / 16;
    const int tail_halves = (int)((bytes - vecs * 16) / 2);
    if (vecs == 0 && tail_halves == 0) return hipSuccess;
    int64_t grid = (vecs + (int64_t)kThreads * 4 - 1) / ((int64_t)kThreads * 4);
    if (grid > kTargetGroups) grid = kTargetGroups;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       (const uint4*)src, (uint4*)dst, vecs,
                       (const uint16_t*)((const char*)src + vecs * 16), (uint16_t*)((char*)dst + vecs * 16),
                       tail_halves);
    return hipGetLastError();
}

hipError_t launch_mse_calibrate(const MseArgs& a, hipStream_t stream)
{
    if (a.B <= 0 || a.elems <= 0) return hipSuccess;
    const int groups = groups_for(a.B, a.elems >> 4, kThreads);
    const dim3 grid((unsigned)(groups * a.B));
    if (a.bf16) hipLaunchKernelGGL(mse_kernel<true>, grid, dim3(kThreads), 0, stream, a, groups);
    else hipLaunchKernelGGL(mse_kernel<false>, grid, dim3(kThreads), 0, stream, a, groups);
    return hipGetLastError();
}

} // namespace qad
