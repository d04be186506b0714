// Fused KL(teacher || student) forward + backward over the vocabulary for
// gfx950 ([Nano] "Von QAT zu QAD": the student is trained to match the frozen
// teacher's output distribution; [Qwen] "3. QAD": logits are compared
// element-wise over the vocabulary and dense fp32 copies of them do not fit,
// so the loss streams bf16 logits and never materialises probabilities).
//
// One workgroup per token row.  Pass 1 streams the row once and keeps, per
// lane, an online (max, sum) pair for teacher and student plus the
// teacher-weighted sum of (t - s), in base 2 (v_exp_f32 computes 2^x; logits
// are scaled by log2(e)/T inside one FMA with the running max).  A workgroup
// reduction merges the lanes.  Pass 2 re-reads the row and writes the gradient
// (q - p) * grad_scale / T with q = 2^(c s - m_s) / Z_s (and p alike): the
// normaliser is a multiply, so the exponent never carries the rounding of a
// large log-sum-exp.  Per-row losses go to row_loss; a single-group
// kernel sums them in a fixed order (binary64) for the mean, so the result
// never depends on scheduling.
#include "qad_device.h"
#include "qad_internal.h"

namespace qad {
namespace {

constexpr int kKlThreads = 1024;
constexpr float kLog2e = 0x1.715476p+0f;  // RN(log2(e))
constexpr float kLn2 = 0x1.62e430p-1f;    // RN(ln(2))

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

struct Stats {
    float mt, zt, at, ms, zs;
};

// merge two partial (max, sum) states; equal maxima (also both -inf) need no
// rescaling, which keeps empty partials from producing 0 * inf
__device__ __forceinline__ Stats merge(const Stats& a, const Stats& b)
{
    Stats r;
    r.mt = fmaxf(a.mt, b.mt);
    const float fa = a.mt == r.mt ? 1.0f : exp2_hw(a.mt - r.mt);
    const float fb = b.mt == r.mt ? 1.0f : exp2_hw(b.mt - r.mt);
    r.zt = a.zt * fa + b.zt * fb;
    r.at = a.at * fa + b.at * fb;
    r.ms = fmaxf(a.ms, b.ms);
    const float ga = a.ms == r.ms ? 1.0f : exp2_hw(a.ms - r.ms);
    const float gb = b.ms == r.ms ? 1.0f : exp2_hw(b.ms - r.ms);
    r.zs = a.zs * ga + b.zs * gb;
    return r;
}

__device__ __forceinline__ Stats shfl_xor_stats(const Stats& s, int o)
{
    Stats r;
    r.mt = __shfl_xor(s.mt, o, 64);
    r.zt = __shfl_xor(s.zt, o, 64);
    r.at = __shfl_xor(s.at, o, 64);
    r.ms = __shfl_xor(s.ms, o, 64);
    r.zs = __shfl_xor(s.zs, o, 64);
    return r;
}

template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t unit, float (&v)[8])
{
    if constexpr (BF16) {
        const uint4 w = reinterpret_cast<const uint4*>(base)[unit];
        v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
        v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(base) + 2 * unit;
        const uint4 w0 = p[0], w1 = p[1];
        v[0] = as_f(w0.x); v[1] = as_f(w0.y); v[2] = as_f(w0.z); v[3] = as_f(w0.w);
        v[4] = as_f(w1.x); v[5] = as_f(w1.y); v[6] = as_f(w1.z); v[7] = as_f(w1.w);
    }
}

__device__ __forceinline__ float max8(const float (&v)[8])
{
    return fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
}

// fold one unit of 8 teacher / student logits into the lane's running state
__device__ __forceinline__ void accumulate(Stats& st, const float (&t)[8], const float (&s)[8], float c)
{
    const float nmt = fmaxf(st.mt, max8(t) * c);
    const float nms = fmaxf(st.ms, max8(s) * c);
    const float ft = st.mt == nmt ? 1.0f : exp2_hw(st.mt - nmt);
    const float fs = st.ms == nms ? 1.0f : exp2_hw(st.ms - nms);
    st.mt = nmt;
    st.ms = nms;
    float et[8], es[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        et[i] = exp2_hw(__builtin_fmaf(t[i], c, -nmt));
        es[i] = exp2_hw(__builtin_fmaf(s[i], c, -nms));
    }
    const float pz = ((et[0] + et[1]) + (et[2] + et[3])) + ((et[4] + et[5]) + (et[6] + et[7]));
    const float qz = ((es[0] + es[1]) + (es[2] + es[3])) + ((es[4] + es[5]) + (es[6] + es[7]));
    float pa = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) pa = __builtin_fmaf(et[i], t[i] - s[i], pa);
    st.zt = st.zt * ft + pz;
    st.at = st.at * ft + pa;
    st.zs = st.zs * fs + qz;
}

template <bool BF16_IN, int GRAD> // GRAD: 0 none, 1 bf16, 2 fp32
__global__ __launch_bounds__(kKlThreads) void kl_row_kernel(KlArgs a, float c, float inv_t, float gmul)
{
    const int64_t row = blockIdx.x;
    const int64_t units = a.vocab >> 3;
    const int64_t ubase = row * units;
    const int tid = threadIdx.x;

    Stats st = {-__builtin_inff(), 0.0f, 0.0f, -__builtin_inff(), 0.0f};
    int64_t u = tid;
    for (; u + kKlThreads < units; u += 2 * kKlThreads) {
        float t0[8], s0[8], t1[8], s1[8];
        load8<BF16_IN>(a.teacher, ubase + u, t0);
        load8<BF16_IN>(a.student, ubase + u, s0);
        load8<BF16_IN>(a.teacher, ubase + u + kKlThreads, t1);
        load8<BF16_IN>(a.student, ubase + u + kKlThreads, s1);
        accumulate(st, t0, s0, c);
        accumulate(st, t1, s1, c);
    }
    if (u < units) {
        float t0[8], s0[8];
        load8<BF16_IN>(a.teacher, ubase + u, t0);
        load8<BF16_IN>(a.student, ubase + u, s0);
        accumulate(st, t0, s0, c);
    }

    // workgroup reduction: waves by xor-shuffles, then the 16 wave results
    for (int o = 32; o > 0; o >>= 1) st = merge(st, shfl_xor_stats(st, o));
    __shared__ Stats part[kKlThreads / 64];
    __shared__ float fin[4];
    if ((tid & 63) == 0) part[tid >> 6] = st;
    __syncthreads();
    if (tid < 64) {
        Stats w = tid < kKlThreads / 64 ? part[tid]
                                        : Stats{-__builtin_inff(), 0.0f, 0.0f, -__builtin_inff(), 0.0f};
        for (int o = 8; o > 0; o >>= 1) w = merge(w, shfl_xor_stats(w, o));
        if (tid == 0) {
            // KL = E_p[t - s]/T - (LSE_t - LSE_s), LSE in log2 units m + log2 Z
            fin[0] = w.mt;
            fin[1] = w.ms;
            fin[2] = gmul / w.zt;
            fin[3] = gmul / w.zs;
            const float kl = (w.at / w.zt) * inv_t - kLn2 * ((w.mt - w.ms) + log2f(w.zt / w.zs));
            a.row_loss[row] = kl;
        }
    }
    if constexpr (GRAD == 0) return;
    __syncthreads();
    const float mt = fin[0], ms = fin[1], wt = fin[2], ws = fin[3];
    for (u = tid; u < units; u += kKlThreads) {
        float t[8], s[8], g[8];
        load8<BF16_IN>(a.teacher, ubase + u, t);
        load8<BF16_IN>(a.student, ubase + u, s);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float eq = exp2_hw(__builtin_fmaf(s[i], c, -ms));
            const float ep = exp2_hw(__builtin_fmaf(t[i], c, -mt));
            g[i] = __builtin_fmaf(eq, ws, -(ep * wt));
        }
        if constexpr (GRAD == 1) {
            reinterpret_cast<uint4*>(a.grad)[ubase + u] =
                make_uint4(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                           pack_bf16x2(g[6], g[7]));
        } else {
            float4* p = reinterpret_cast<float4*>(a.grad) + 2 * (ubase + u);
            p[0] = make_float4(g[0], g[1], g[2], g[3]);
            p[1] = make_float4(g[4], g[5], g[6], g[7]);
        }
    }
}

// mean of the per-row losses: fixed assignment of rows to lanes, binary64
// accumulation, fixed reduction tree
__global__ __launch_bounds__(kKlThreads) void kl_mean_kernel(const float* row_loss, int64_t rows, float* loss_out)
{
    __shared__ double part[kKlThreads];
    double acc = 0.0;
    for (int64_t r = threadIdx.x; r < rows; r += kKlThreads) acc += (double)row_loss[r];
    part[threadIdx.x] = acc;
    __syncthreads();
    for (int w = kKlThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) loss_out[0] = rows > 0 ? (float)(part[0] / (double)rows) : 0.0f;
}

} // namespace

hipError_t launch_kl(const KlArgs& a, hipStream_t stream)
{
    if (a.tokens > 0 && a.vocab > 0) {
        const float c = kLog2e / a.temperature;
        const float inv_t = 1.0f / a.temperature;
        const float gmul = a.grad_scale / a.temperature;
        const dim3 grid((unsigned)a.tokens), block(kKlThreads);
        if (a.bf16_in) {
            if (!a.grad) hipLaunchKernelGGL((kl_row_kernel<true, 0>), grid, block, 0, stream, a, c, inv_t, gmul);
            else if (a.grad_bf16) hipLaunchKernelGGL((kl_row_kernel<true, 1>), grid, block, 0, stream, a, c, inv_t, gmul);
            else hipLaunchKernelGGL((kl_row_kernel<true, 2>), grid, block, 0, stream, a, c, inv_t, gmul);
        } else {
            if (!a.grad) hipLaunchKernelGGL((kl_row_kernel<false, 0>), grid, block, 0, stream, a, c, inv_t, gmul);
            else if (a.grad_bf16) hipLaunchKernelGGL((kl_row_kernel<false, 1>), grid, block, 0, stream, a, c, inv_t, gmul);
            else hipLaunchKernelGGL((kl_row_kernel<false, 2>), grid, block, 0, stream, a, c, inv_t, gmul);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kl_mean_kernel, dim3(1), dim3(kKlThreads), 0, stream, a.row_loss, a.tokens, a.loss_out);
    return hipGetLastError();
}

} // namespace qad
