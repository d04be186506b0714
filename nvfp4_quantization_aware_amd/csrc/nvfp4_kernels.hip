// NVFP4 simulated-quantization kernels for gfx950: tensor amax, quantize /
// dequantize with dynamic or frozen scales, the straight-through copy and the
// MSE block-scale search.  Page legend and numerical conventions: see
// include/libqad.h.  Nothing here is a contraction, so there is no MFMA; every
// kernel streams HBM with 16-byte non-temporal loads and stores, and every
// workgroup owns one small contiguous chunk of a tensor (this access pattern
// measured fastest on MI355X: ~6.2 TB/s copy, ~7.1 TB/s read).
//
// Dynamic scales need the tensor amax before any element can be coded.  For
// tensors whose chunks fit on the chip at once (an MoE expert: 16 MiB), the
// quantizer reads the tensor ONCE: each workgroup keeps its chunk in
// registers, publishes the chunk maximum, waits for the tensor's maximum and
// codes from registers (see "one-pass protocol" below).  Larger tensors take
// two passes (amax kernel, then quantizer).
#include "qad_device.h"
#include "qad_internal.h"

namespace qad {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// RN(1/6) in binary32 (0x3E2AAAAB)
constexpr float kRcp6 = 0x1.555556p-3f;
// Tensor scales at or above this use the reciprocal division (its validity
// range); smaller ones take IEEE division everywhere.
constexpr float kFastMinScale = 0x1p-80f;
constexpr int kQThreads = 256;
// The one-pass wait is bounded: after QuantizeArgs::wait_ticks ticks of the
// 100 MHz wall clock (20 ms by default) a workgroup stops waiting and
// computes what it waited for itself.

__device__ __forceinline__ v4u ldnt(const void* p, int64_t i) { return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p) + i); }
__device__ __forceinline__ void stnt(void* p, int64_t i, v4u v) { __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(p) + i); }
__device__ __forceinline__ void stnt32(void* p, int64_t i, uint32_t v) { __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p) + i); }
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef short fp8x2_t __attribute__((ext_vector_type(2)));   // two FP8 codes in a 32-bit register half
__device__ __forceinline__ void stnt64(void* p, int64_t i, uint32_t lo, uint32_t hi) { __builtin_nontemporal_store(v2u{lo, hi}, reinterpret_cast<v2u*>(p) + i); }

// ---- agent-scope atomics used by the one-pass protocol ---------------------
__device__ __forceinline__ uint32_t a_load(const uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void a_store(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ uint32_t a_max(uint32_t* p, uint32_t v) { return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ uint32_t a_add(uint32_t* p, uint32_t v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// compare-and-swap: true when *p was `expected` and now holds `desired`
__device__ __forceinline__ bool a_cas(uint32_t* p, uint32_t expected, uint32_t desired)
{
    return __hip_atomic_compare_exchange_strong(p, &expected, desired, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until the value returned by a preceding atomic has arrived, i.e. the
// atomic has been performed, before any later memory operation is issued.
__device__ __forceinline__ void completed(uint32_t v) { asm volatile("" ::"v"(v) : "memory"); }

// units of 8 elements per lane in one chunk: 128 bytes of input per lane
template <bool BF16> struct Chunk {
    static constexpr int U = BF16 ? 8 : 4;
    static constexpr int64_t UNITS = (int64_t)kQThreads * U;
};

// raw input of one unit (8 elements): one 16-byte vector for bf16, two for fp32
template <bool BF16> struct Raw;
template <> struct Raw<true> { v4u a; };
template <> struct Raw<false> { v4u a, b; };

template <bool BF16>
__device__ __forceinline__ Raw<BF16> load_raw(const void* x, int64_t unit, bool valid)
{
    Raw<BF16> r;
    if constexpr (BF16) {
        r.a = valid ? ldnt(x, unit) : v4u{0u, 0u, 0u, 0u};
    } else {
        r.a = valid ? ldnt(x, 2 * unit) : v4u{0u, 0u, 0u, 0u};
        r.b = valid ? ldnt(x, 2 * unit + 1) : v4u{0u, 0u, 0u, 0u};
    }
    return r;
}

template <bool BF16>
__device__ __forceinline__ void unpack(const Raw<BF16>& r, float (&e)[8])
{
    if constexpr (BF16) {
        e[0] = bf_lo(r.a.x); e[1] = bf_hi(r.a.x); e[2] = bf_lo(r.a.y); e[3] = bf_hi(r.a.y);
        e[4] = bf_lo(r.a.z); e[5] = bf_hi(r.a.z); e[6] = bf_lo(r.a.w); e[7] = bf_hi(r.a.w);
    } else {
        e[0] = as_f(r.a.x); e[1] = as_f(r.a.y); e[2] = as_f(r.a.z); e[3] = as_f(r.a.w);
        e[4] = as_f(r.b.x); e[5] = as_f(r.b.y); e[6] = as_f(r.b.z); e[7] = as_f(r.b.w);
    }
}

// largest magnitude of a unit as binary32 bits: magnitudes of finite values
// order like their bit patterns with the sign cleared (integer max: exact and
// independent of evaluation order)
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

template <bool BF16>
__device__ __forceinline__ uint32_t unit_absmax(const Raw<BF16>& r)
{
    if constexpr (BF16) {
        // both bf16 halves of each word at once (packed 16-bit integer max)
        us2 m = __builtin_elementwise_max(__builtin_bit_cast(us2, r.a.x & 0x7FFF7FFFu),
                                          __builtin_bit_cast(us2, r.a.y & 0x7FFF7FFFu));
        m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, r.a.z & 0x7FFF7FFFu));
        m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, r.a.w & 0x7FFF7FFFu));
        return umax((uint32_t)m.x, (uint32_t)m.y) << 16;
    } else {
        return umax(umax(umax(r.a.x & 0x7FFFFFFFu, r.a.y & 0x7FFFFFFFu), umax(r.a.z & 0x7FFFFFFFu, r.a.w & 0x7FFFFFFFu)),
                    umax(umax(r.b.x & 0x7FFFFFFFu, r.b.y & 0x7FFFFFFFu), umax(r.b.z & 0x7FFFFFFFu, r.b.w & 0x7FFFFFFFu)));
    }
}

// workgroup maximum (result valid in every thread)
__device__ __forceinline__ uint32_t group_max(uint32_t m, uint32_t* red)
{
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    uint32_t r = red[0];
    for (int w = 1; w < kQThreads / 64; ++w) r = umax(r, red[w]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ float tensor_scale_of(uint32_t amax_bits)
{
    const float amax = as_f(amax_bits);
    return amax > 0.0f ? amax / 2688.0f : 1.0f;
}

// FP8 (E4M3) per-tensor scale: the amax onto the E4M3 maximum 448
__device__ __forceinline__ float fp8_scale_of(uint32_t amax_bits)
{
    const float amax = as_f(amax_bits);
    return amax > 0.0f ? amax / 448.0f : 1.0f;
}

// ---------------------------------------------------------------------------
// Per-tensor record in the workspace, used by the amax publication.
//   word 0: tensor amax (binary32 bits), word 1: completed sub-groups
//   sub-group s (16 consecutive chunks): words 32+32s (max), 33+32s (arrivals),
//     34+32s (maximum found by a fallback scan | 0x80000000), 35+32s (claim
//     of that scan)
//   broadcast slot of chunk j: word 32 + 32*nsub + 16*j (amax | 0x80000000)
// Every field sits on its own 64- or 128-byte line so that no address sees
// more than ~16 atomics or one poller.  Records are zeroed before each launch.
// ---------------------------------------------------------------------------
struct Record {
    uint32_t* w;
    int64_t chunks, nsub;
    __device__ Record(uint32_t* base, int64_t b, int64_t P)
        : w(base + b * record_words(P)), chunks(P), nsub((P + 15) / 16) {}
    __device__ uint32_t* slot(int64_t j) const { return w + 32 + 32 * nsub + 16 * j; }
};

// Publish chunk j's maximum m (thread 0 only).  Returns true in exactly one
// chunk: the one whose arrival completes the tensor; record word 0 then holds
// the tensor amax.  Order is carried by completion: each atomic's returned
// value is awaited before the next is issued, so an arrival count is only
// ever observed after the maxima it accounts for have been performed.
__device__ bool publish_max(const Record& r, int64_t j, uint32_t m)
{
    const int64_t s = j / 16;
    const uint32_t members = (uint32_t)(r.chunks - s * 16 < 16 ? r.chunks - s * 16 : 16);
    uint32_t* sw = r.w + 32 + 32 * s;
    completed(a_max(sw, m));
    const uint32_t k = a_add(sw + 1, 1u);
    completed(k);
    if (k != members - 1) return false;
    const uint32_t sub = a_load(sw);
    completed(a_max(r.w, sub));
    const uint32_t k2 = a_add(r.w + 1, 1u);
    completed(k2);
    return k2 == (uint32_t)r.nsub - 1;
}

// ---------------------------------------------------------------------------
// Per-tensor table in LDS: effective scale dec(c) * s_g of every E4M3 code c
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

// x / s correctly rounded for x >= 0 (+0 included; s = 0 gives +0)
template <bool FAST>
__device__ __forceinline__ float quotient_pos(float x, float s, float r)
{
    if constexpr (FAST) return div_rcp(x, s, r);
    else return s > 0.0f ? x / s : 0.0f;
}

// x / s correctly rounded, with x's sign bit (s = 0 gives a signed zero)
template <bool FAST>
__device__ __forceinline__ float quotient(float x, float s, float r)
{
    if constexpr (FAST) return div_rcp_signed(x, s, r);
    else return __builtin_copysignf(quotient_pos<FAST>(__builtin_fabsf(x), s, r), x);
}

// Code one unit (half a block; the lane pair owns the block).  Returns the
// block's scale code; writes the 8 packed codes (even element in the low
// nibble) and the 8 bf16 outputs y = bf16(dec(code) * s_eff).
template <bool FROZEN, bool FAST>
__device__ __forceinline__ uint32_t quantize_unit(const float (&e)[8], uint32_t unit_max, uint32_t frozen_code,
                                                  const ScaleTable& tab, float s_g, float rcp_g, uint32_t& code,
                                                  uint32_t (&yw)[4])
{
    const uint32_t m = umax(unit_max, swap_pair(unit_max)); // block amax (binary32 bits)
    uint32_t sb = FROZEN ? frozen_code : block_scale_code<FAST>(as_f(m), s_g, rcp_g);
    sb &= 127u;
    const float s = tab.seff[sb], r = tab.rcp[sb];
    float q[8];
    if constexpr (FROZEN && FAST) {
        // A frozen scale may be far below an element: x r would overflow and
        // the reciprocal scheme turn it into NaN.  Every quotient >= 8
        // saturates to the same code, so x is first clamped to +-8 s (exact;
        // signed zeros and everything below the bound pass unchanged).  A
        // dynamic scale keeps every quotient below 12, and IEEE division
        // (small tensor scales) saturates by itself.
        const float lim = s > 0.0f ? 8.0f * s : 0x1.fffffep127f;
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = quotient<FAST>(__builtin_amdgcn_fmed3f(e[i], -lim, lim), s, r);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = quotient<FAST>(e[i], s, r);
    }
    uint32_t c = 0;
    c = fp4_encode_pair<0>(c, q[0], q[1]);
    c = fp4_encode_pair<1>(c, q[2], q[3]);
    c = fp4_encode_pair<2>(c, q[4], q[5]);
    c = fp4_encode_pair<3>(c, q[6], q[7]);
    code = c;
    float g[8];
    fp4_decode_pair<0>(c, g[0], g[1]);
    fp4_decode_pair<1>(c, g[2], g[3]);
    fp4_decode_pair<2>(c, g[4], g[5]);
    fp4_decode_pair<3>(c, g[6], g[7]);
#pragma unroll
    for (int i = 0; i < 8; i += 2) yw[i >> 1] = pack_bf16x2(g[i] * s, g[i + 1] * s);
    return sb;
}

// FP8 (E4M3) per-tensor QDQ of one unit of 8 elements ([Qwen] "3. QAD":
// attention projections FP8 W8A8, KV cache FP8): code = sign | E4M3(|x|/s),
// nearest even, saturating at 448; y = bf16(dec(code) * s).  Codes are the 8
// bytes of the unit in element order.  The quotient is clamped to +-448 and
// converted by gfx950's FP8 instructions with unit scale (nearest even on
// every input up to 448 in magnitude, signs and subnormals included; beyond
// 464 they give NaN, hence the clamp); decoding is the reverse instruction.
// A frozen scale may lie far below an element, where x r overflows: frozen
// elements are first clamped to +-1024 s (exact), which saturates the same.
template <bool FAST, bool FROZEN>
__device__ __forceinline__ void fp8_unit(const float (&e)[8], float s, float r, uint32_t (&code)[2], uint32_t (&yw)[4])
{
    float q[8];
    const float lim = FROZEN && FAST ? 1024.0f * s : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x = FROZEN && FAST ? __builtin_amdgcn_fmed3f(e[i], -lim, lim) : e[i];
        q[i] = __builtin_amdgcn_fmed3f(quotient<FAST>(x, s, r), -448.0f, 448.0f);
    }
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        fp8x2_t lo = {0, 0};
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, q[4 * w], q[4 * w + 1], 1.0f, false);
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, q[4 * w + 2], q[4 * w + 3], 1.0f, true);
        code[w] = __builtin_bit_cast(uint32_t, lo);
        const auto g01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(code[w], 1.0f, false);
        const auto g23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(code[w], 1.0f, true);
        yw[2 * w] = pack_bf16x2(g01[0] * s, g01[1] * s);
        yw[2 * w + 1] = pack_bf16x2(g23[0] * s, g23[1] * s);
    }
}

enum { MODE_FROZEN = 0, MODE_AMAX = 1, MODE_ONEPASS = 2 };

template <bool BF16, int MODE, bool FAST, bool FP8>
__device__ __forceinline__ void code_chunk(const QuantizeArgs& a, const Raw<BF16> (&raw)[Chunk<BF16>::U],
                                           const uint32_t (&unit_max)[Chunk<BF16>::U], int64_t ubase, int64_t u0,
                                           int64_t units, const ScaleTable& tab, float s_g)
{
    const float rcp_g = 1.0f / s_g;
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < Chunk<BF16>::U; ++k) {
        const int64_t u = u0 + k * kQThreads + t;
        const bool valid = u < units;
        float e[8];
        unpack<BF16>(raw[k], e);
        if constexpr (FP8) {
            uint32_t code[2], yw[4];
            fp8_unit<FAST, MODE == MODE_FROZEN>(e, s_g, rcp_g, code, yw);
            if (valid) {
                if (a.y) stnt(a.y, ubase + u, v4u{yw[0], yw[1], yw[2], yw[3]});
                if (a.codes) stnt64(a.codes, ubase + u, code[0], code[1]);
            }
            continue;
        }
        uint32_t frozen_code = 0;
        if constexpr (MODE == MODE_FROZEN) frozen_code = valid ? a.scales_in[(ubase + u) >> 1] : 0u;
        uint32_t code, yw[4];
        const uint32_t sb = quantize_unit<MODE == MODE_FROZEN, FAST>(e, unit_max[k], frozen_code, tab, s_g, rcp_g,
                                                                     code, yw);
        if (valid) {
            if (a.y) stnt(a.y, ubase + u, v4u{yw[0], yw[1], yw[2], yw[3]});
            if (a.codes) stnt32(a.codes, ubase + u, code);
            if (a.scales_out && !(t & 1)) a.scales_out[(ubase + u) >> 1] = (uint8_t)sb;
        }
    }
}

// Tensor amax after a timed-out wait (exact, so it equals the published one),
// reading only what has not been published.  A sub-group whose arrivals are
// complete contributes its published maximum.  Each unfinished sub-group is
// scanned (its 16 chunks of input) by the one workgroup that claims it.  A
// workgroup claims one sub-group at a time, looking first at its own
// (`first`) and then onward, scans it and looks again, so that the scans of
// many timed-out workgroups spread over the sub-groups; when none is left to
// claim, wave 0 collects every sub-group's maximum, waiting where another
// workgroup's scan is still running -- that scan needs nothing from anyone,
// so the wait ends.  However many workgroups time out, each byte of the
// tensor is read at most once more.  Returns the amax; *scanned tells whether
// this workgroup scanned anything.  `sh` is three words of LDS.
template <bool BF16>
__device__ uint32_t fallback_amax(const Record& rec, const void* x, int64_t ubase, int64_t units, int first,
                                  uint32_t* red, uint32_t* sh, bool* scanned)
{
    constexpr int64_t kSubUnits = 16 * Chunk<BF16>::UNITS;
    const int t = threadIdx.x;
    const int nsub = (int)rec.nsub, chunks = (int)rec.chunks;   // at most 64 and 1024 on this path
    *scanned = false;
    for (;;) {
        if (t == 0) {
            int claim = -1;
            int sg = first;
            for (int i = 0; i < nsub && claim < 0; ++i, sg = sg + 1 == nsub ? 0 : sg + 1) {
                uint32_t* sw = rec.w + 32 + 32 * sg;
                const uint32_t members = (uint32_t)(chunks - sg * 16 < 16 ? chunks - sg * 16 : 16);
                if (a_load(sw + 3) != 0u || a_load(sw + 1) == members) continue;   // claimed, or complete
                if (a_cas(sw + 3, 0u, 1u)) claim = sg;
            }
            sh[0] = (uint32_t)(claim + 1);
        }
        __syncthreads();
        const int sg = (int)sh[0] - 1;
        __syncthreads();
        if (sg < 0) break;
        *scanned = true;
        const int64_t u0 = sg * kSubUnits;
        const int n = (int)((u0 + kSubUnits < units ? u0 + kSubUnits : units) - u0);
        uint32_t m = 0;
        for (int u = t; u < n; u += kQThreads) m = umax(m, unit_absmax<BF16>(load_raw<BF16>(x, ubase + u0 + u, true)));
        m = group_max(m, red);
        if (t == 0) a_store(rec.w + 32 + 32 * sg + 2, m | 0x80000000u);
    }
    if (t < 64) {
        uint32_t am = 0;
        for (int sg = t; sg < nsub; sg += 64) {
            uint32_t* sw = rec.w + 32 + 32 * sg;
            const uint32_t members = (uint32_t)(chunks - sg * 16 < 16 ? chunks - sg * 16 : 16);
            for (;;) {
                if (a_load(sw + 1) == members) {
                    am = umax(am, a_load(sw));
                    break;
                }
                const uint32_t sc = a_load(sw + 2);
                if (sc & 0x80000000u) {
                    am = umax(am, sc & 0x7FFFFFFFu);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        am = wave_max_u32(am);
        if (t == 0) sh[2] = am;
    }
    __syncthreads();
    return sh[2];
}

// ---------------------------------------------------------------------------
// The quantizer.  One workgroup per chunk of Chunk::UNITS units (32 KiB of
// bf16 / fp32 input); chunk c is chunk j = c % P of tensor b = c / P.  A lane
// holds units u0 + k*256 + lane, so lanes 2i and 2i+1 hold the two halves of a
// block.  s_g comes from the frozen input (MODE_FROZEN), from the amax kernel
// (MODE_AMAX) or from the one-pass protocol (MODE_ONEPASS):
//   1. every workgroup reduces its chunk's maximum and publishes it
//      (publish_max); the workgroup completing the tensor writes the amax
//      into every chunk's broadcast slot;
//   2. each workgroup waits on its own slot, then codes from registers.
// Progress: workgroups are dispatched in order on each XCD and the host only
// takes this path when at most half of the resident workgroups are needed to
// hold one tensor, so the chunks a waiting workgroup depends on are always
// resident or finished.  The wait is nevertheless bounded; on time-out the
// workgroup computes the amax itself (exact, so the result is unchanged).
// ---------------------------------------------------------------------------
template <bool BF16, int MODE, bool FP8>
__global__ __launch_bounds__(kQThreads) void quantize_kernel(QuantizeArgs a, int64_t P, uint32_t* ws)
{
    using CH = Chunk<BF16>;
    __shared__ ScaleTable tab;
    __shared__ uint32_t red[kQThreads / 64];
    __shared__ uint32_t sh_bcast, sh_amax, sh_fb[3];
    const int64_t c = blockIdx.x;
    const int64_t b = c / P, j = c - b * P;
    const int64_t units = a.elems >> 3;
    const int64_t ubase = b * units;
    const int64_t u0 = j * CH::UNITS;
    const int t = threadIdx.x;

    // One pass: the chunk's loads are issued at the highest wave priority, so
    // that the arbiter serves a wave that is starting its loads before the
    // resident waves that are coding a chunk; that gets more bytes in flight
    // while other workgroups wait on their tensor's maximum (the 128-expert
    // batch: 0.815 -> 0.770 ms; the other modes, the amax pass and the copy
    // measured no better or worse with it).
    if constexpr (MODE == MODE_ONEPASS) __builtin_amdgcn_s_setprio(3);
    Raw<BF16> raw[CH::U];
#pragma unroll
    for (int k = 0; k < CH::U; ++k) {
        const int64_t u = u0 + k * kQThreads + t;
        raw[k] = load_raw<BF16>(a.x, ubase + u, u < units);
    }
    if constexpr (MODE == MODE_ONEPASS) __builtin_amdgcn_s_setprio(0);
    float s_g;
    if constexpr (MODE == MODE_FROZEN) {
        s_g = a.tscale_in[b];
    } else if constexpr (MODE == MODE_AMAX) {
        const uint32_t am = Record(ws, b, P).w[0]; // written by amax_kernel (same chunking)
        s_g = FP8 ? fp8_scale_of(am) : tensor_scale_of(am);
    } else {
        const Record rec(ws, b, P);
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < CH::U; ++k) m = umax(m, unit_absmax<BF16>(raw[k]));
        m = group_max(m, red);
        if (t == 0) sh_bcast = publish_max(rec, j, m) ? (a_load(rec.w) | 0x80000000u) : 0u;
        __syncthreads();
        const uint32_t bc = sh_bcast;
        if (bc)
            for (int64_t i = t; i < P; i += kQThreads) a_store(rec.slot(i), bc);
        if (t == 0) {
            const uint64_t t0 = wall_clock64();
            uint32_t w;
            while (!((w = a_load(rec.slot(j))) & 0x80000000u)) {
                __builtin_amdgcn_s_sleep(8);
                if (wall_clock64() - t0 > a.wait_ticks) break;
            }
            sh_amax = w;
        }
        __syncthreads();
        uint32_t am = sh_amax;
        if (!(am & 0x80000000u)) {
            // timed out: the amax from what is published plus scans of the rest
            bool scanned;
            am = fallback_amax<BF16>(rec, a.x, ubase, units, (int)(j / 16), red, sh_fb, &scanned) | 0x80000000u;
            if (scanned)   // a workgroup that scanned broadcasts, so that no chunk waits any longer
                for (int64_t i = t; i < P; i += kQThreads) a_store(rec.slot(i), am);
            // the chunk is read again rather than held across this rare path,
            // which leaves the fallback the registers the chunk occupied
#pragma unroll
            for (int k = 0; k < CH::U; ++k) {
                const int64_t u = u0 + k * kQThreads + t;
                raw[k] = load_raw<BF16>(a.x, ubase + u, u < units);
            }
        }
        s_g = FP8 ? fp8_scale_of(am & 0x7FFFFFFFu) : tensor_scale_of(am & 0x7FFFFFFFu);
    }
    if (!FP8) build_table(tab, s_g);
    if (j == 0 && t == 0 && a.tscale_out) a.tscale_out[b] = s_g;
    // each unit's largest magnitude (binary32 bits), from the packed data
    uint32_t unit_max[CH::U];
#pragma unroll
    for (int k = 0; k < CH::U; ++k) unit_max[k] = unit_absmax<BF16>(raw[k]);
    __syncthreads();
    if (s_g >= kFastMinScale) code_chunk<BF16, MODE, true, FP8>(a, raw, unit_max, ubase, u0, units, tab, s_g);
    else code_chunk<BF16, MODE, false, FP8>(a, raw, unit_max, ubase, u0, units, tab, s_g);
}

// ---------------------------------------------------------------------------
// Tensor amax for the two-pass path and nvfp4_amax: one workgroup per chunk,
// hierarchical publication into the tensor record (word 0 ends as the amax).
// `vecs` counts 16-byte vectors per tensor.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kQThreads) void amax_kernel(const void* x, int64_t vecs, int64_t P, uint32_t* ws)
{
    __shared__ uint32_t red[kQThreads / 64];
    constexpr int64_t kVecs = (int64_t)kQThreads * 8; // 32 KiB per chunk
    const int64_t c = blockIdx.x, b = c / P, j = c - b * P;
    const int64_t v0 = j * kVecs, base = b * vecs;
    uint32_t m = 0;
    v4u v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int64_t i = v0 + k * kQThreads + threadIdx.x;
        v[k] = i < vecs ? ldnt(x, base + i) : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if constexpr (BF16) {
            Raw<true> r{v[k]};
            m = umax(m, unit_absmax<true>(r));
        } else {
            m = umax(m, umax(umax(v[k].x & 0x7FFFFFFFu, v[k].y & 0x7FFFFFFFu), umax(v[k].z & 0x7FFFFFFFu, v[k].w & 0x7FFFFFFFu)));
        }
    }
    m = group_max(m, red);
    if (threadIdx.x == 0) publish_max(Record(ws, b, P), j, m);
}

// record word 0 of every tensor -> out[b] (nvfp4_amax result)
__global__ void amax_out_kernel(const uint32_t* ws, int64_t B, int64_t P, uint32_t* out)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) out[b] = ws[b * record_words(P)];
}

__global__ void fill_u32_kernel(uint32_t* out, int64_t n, uint32_t v)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) out[i] = v;
}

__global__ void copy_u32_kernel(const uint32_t* src, uint32_t* dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// Straight-through backward: chunked 16-byte non-temporal copy (16 KiB per
// workgroup) plus a tail of up to seven 16-bit halves.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kQThreads) void copy_kernel(const void* __restrict__ src, void* __restrict__ dst,
                                                         int64_t vecs, const uint16_t* __restrict__ src_tail,
                                                         uint16_t* __restrict__ dst_tail, int tail_halves)
{
    const int64_t v0 = (int64_t)blockIdx.x * (kQThreads * 4);
    v4u v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t i = v0 + k * kQThreads + threadIdx.x;
        if (i < vecs) v[k] = ldnt(src, i);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t i = v0 + k * kQThreads + threadIdx.x;
        if (i < vecs) stnt(dst, i, v[k]);
    }
    if (blockIdx.x == 0 && threadIdx.x < tail_halves) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}

// ---------------------------------------------------------------------------
// Clipped straight-through backward ([Lightning] "量化尺度处理策略": with
// frozen scales only the weights train).  grad_x = grad_y where the element
// lies inside the range its block represents, |x| <= 6 * s_eff, and +0 where
// the quantizer saturates; s_eff = dec(s_b) * s_g as in the forward.  The
// test is exact: fma(-6, s_eff, |x|) rounds |x| - 6 * s_eff once, and both
// terms are multiples of 2^-149, so a nonzero difference never rounds to 0
// and the sign is the exact one.  One lane per unit of 8 elements (half a
// block), kClipUnits units per lane strided by the workgroup width, one
// tensor per group of workgroups (uniform tensor scale).
// ---------------------------------------------------------------------------
constexpr int kClipUnits = 4;

template <bool GBF16, bool XBF16>
__global__ __launch_bounds__(kQThreads) void clip_ste_kernel(ClipArgs a, int64_t P)
{
    const int64_t b = blockIdx.x / P;
    const int64_t u0 = (blockIdx.x - b * P) * ((int64_t)kQThreads * kClipUnits);
    const int64_t upt = a.elems >> 3;
    const float s_g = a.tscale[b];
    const void* gy = (const char*)a.grad_y + b * a.elems * (GBF16 ? 2 : 4);
    const void* x = (const char*)a.x + b * a.elems * (XBF16 ? 2 : 4);
    void* gx = (char*)a.grad_x + b * a.elems * (GBF16 ? 2 : 4);
    const uint8_t* sc = a.scales + b * (a.elems >> 4);
    Raw<GBF16> g[kClipUnits];
    Raw<XBF16> xr[kClipUnits];
    uint32_t code[kClipUnits];
#pragma unroll
    for (int k = 0; k < kClipUnits; ++k) {
        const int64_t u = u0 + k * kQThreads + threadIdx.x;
        const bool valid = u < upt;
        g[k] = load_raw<GBF16>(gy, u, valid);
        xr[k] = load_raw<XBF16>(x, u, valid);
        code[k] = valid ? sc[u >> 1] : 0u;
    }
#pragma unroll
    for (int k = 0; k < kClipUnits; ++k) {
        const int64_t u = u0 + k * kQThreads + threadIdx.x;
        if (u >= upt) continue;
        float e[8];
        unpack<XBF16>(xr[k], e);
        const float s = e4m3_decode(code[k] & 127u) * s_g;
        bool keep[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) keep[i] = __builtin_fmaf(-6.0f, s, __builtin_fabsf(e[i])) <= 0.0f;
        if constexpr (GBF16) {
            uint32_t w[4] = {g[k].a.x, g[k].a.y, g[k].a.z, g[k].a.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = (keep[2 * i] ? w[i] & 0xFFFFu : 0u) | (keep[2 * i + 1] ? w[i] & 0xFFFF0000u : 0u);
            stnt(gx, u, v4u{w[0], w[1], w[2], w[3]});
        } else {
            stnt(gx, 2 * u, v4u{keep[0] ? g[k].a.x : 0u, keep[1] ? g[k].a.y : 0u, keep[2] ? g[k].a.z : 0u,
                                keep[3] ? g[k].a.w : 0u});
            stnt(gx, 2 * u + 1, v4u{keep[4] ? g[k].b.x : 0u, keep[5] ? g[k].b.y : 0u, keep[6] ? g[k].b.z : 0u,
                                    keep[7] ? g[k].b.w : 0u});
        }
    }
}

// ---------------------------------------------------------------------------
// Frozen-scale SGD weight step ([Lightning] "量化尺度处理策略": frozen scales
// stay fixed and only the weights move; "训练配置": a constant learning rate
// and clipping of the gradient norm, whose coefficient the caller computed).
// The gradient reaches the weight through the clipped straight-through
// estimator, so a weight the quantizer saturates (|w| > 6 * s_eff, the same
// exact test as above) keeps its value, and every other weight becomes
// fma(-a, g, w) rounded to the weight's dtype, a = lr * clip_coef in
// binary32.  One pass over w and g: the weight is both the quantizer's input
// (for the clip) and the value updated.  Launch shape of the clipped backward.
// ---------------------------------------------------------------------------
template <bool WBF16, bool GBF16>
__global__ __launch_bounds__(kQThreads) void sgd_step_kernel(SgdArgs a, int64_t P)
{
    const int64_t b = blockIdx.x / P;
    const int64_t u0 = (blockIdx.x - b * P) * ((int64_t)kQThreads * kClipUnits);
    const int64_t upt = a.elems >> 3;
    const float s_g = a.tscale[b];
    const float step = a.lr * a.clip_coef;
    const void* w = (const char*)a.w + b * a.elems * (WBF16 ? 2 : 4);
    const void* gr = (const char*)a.grad + b * a.elems * (GBF16 ? 2 : 4);
    void* wo = (char*)a.w_out + b * a.elems * (WBF16 ? 2 : 4);
    const uint8_t* sc = a.scales + b * (a.elems >> 4);
    Raw<WBF16> wr[kClipUnits];
    Raw<GBF16> g[kClipUnits];
    uint32_t code[kClipUnits];
#pragma unroll
    for (int k = 0; k < kClipUnits; ++k) {
        const int64_t u = u0 + k * kQThreads + threadIdx.x;
        const bool valid = u < upt;
        wr[k] = load_raw<WBF16>(w, u, valid);
        g[k] = load_raw<GBF16>(gr, u, valid);
        code[k] = valid ? sc[u >> 1] : 0u;
    }
#pragma unroll
    for (int k = 0; k < kClipUnits; ++k) {
        const int64_t u = u0 + k * kQThreads + threadIdx.x;
        if (u >= upt) continue;
        float e[8], gv[8], r[8];
        unpack<WBF16>(wr[k], e);
        unpack<GBF16>(g[k], gv);
        const float s = e4m3_decode(code[k] & 127u) * s_g;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool keep = __builtin_fmaf(-6.0f, s, __builtin_fabsf(e[i])) <= 0.0f;
            r[i] = keep ? __builtin_fmaf(-step, gv[i], e[i]) : e[i];
        }
        if constexpr (WBF16) {
            stnt(wo, u, v4u{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
                            pack_bf16x2(r[6], r[7])});
        } else {
            stnt(wo, 2 * u, v4u{as_u(r[0]), as_u(r[1]), as_u(r[2]), as_u(r[3])});
            stnt(wo, 2 * u + 1, v4u{as_u(r[4]), as_u(r[5]), as_u(r[6]), as_u(r[7])});
        }
    }
}

// ---------------------------------------------------------------------------
// MSE calibration of the frozen block scales ([Lightning] "量化尺度处理策略").
// One lane per 16-element block.  The candidates amax_b * k_i / 6 rounded to
// E4M3 are non-decreasing in i and, for grids no coarser than k_min/16 per
// step, visit every code between the first and the last candidate's code
// without a gap.  So the search runs over that contiguous code range (at most
// 9 codes for k in [0.5, 1]) instead of all n candidates, and equal errors go
// to the lowest code ("first candidate with strictly smaller error").
// ---------------------------------------------------------------------------
template <bool FAST>
__device__ __forceinline__ float block_error(const float (&e)[16], float s, float r)
{
    // squared error of the block under effective scale s, summed in element
    // order; magnitudes only (|x - dec * s| is symmetric in the sign)
    float q[16], g[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) q[j] = quotient_pos<FAST>(__builtin_fabsf(e[j]), s, r);
#pragma unroll
    for (int j = 0; j < 16; j += 8) {
        uint32_t c = 0;
        c = fp4_encode_pair<0>(c, q[j], q[j + 1]);
        c = fp4_encode_pair<1>(c, q[j + 2], q[j + 3]);
        c = fp4_encode_pair<2>(c, q[j + 4], q[j + 5]);
        c = fp4_encode_pair<3>(c, q[j + 6], q[j + 7]);
        fp4_decode_pair<0>(c, g[j], g[j + 1]);
        fp4_decode_pair<1>(c, g[j + 2], g[j + 3]);
        fp4_decode_pair<2>(c, g[j + 4], g[j + 5]);
        fp4_decode_pair<3>(c, g[j + 6], g[j + 7]);
    }
    float err = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float d = __builtin_fabsf(e[j]) - g[j] * s;
        err = err + d * d;
    }
    return err;
}

// squared error of the block's largest element alone under effective scale
// s, computed exactly as its term inside block_error: a lower bound of the
// block error (a binary32 running sum of non-negative terms never falls
// below any of its terms)
template <bool FAST>
__device__ __forceinline__ float max_term(float amax_b, float s, float r)
{
    const float q = quotient_pos<FAST>(amax_b, s, r);
    float g, unused;
    fp4_decode_pair<0>(fp4_encode_pair<0>(0u, q, 0.0f), g, unused);
    const float d = amax_b - g * s;
    return d * d;
}

template <bool BF16, bool FAST>
__device__ __forceinline__ void calibrate_tensor(const MseArgs& a, int64_t b, int64_t g, int64_t groups,
                                                 const ScaleTable& tab, float s_g)
{
    const int64_t nblk = a.elems >> 4;
    const float rcp_g = 1.0f / s_g;
    const int64_t stride = groups * kQThreads;
    for (int64_t blk = g * kQThreads + threadIdx.x; blk < nblk; blk += stride) {
        const int64_t gb = b * nblk + blk;
        float e[16];
        if constexpr (BF16) {
            const v4u v0 = ldnt(a.w, 2 * gb), v1 = ldnt(a.w, 2 * gb + 1);
            const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int q = 0; q < 8; ++q) { e[2 * q] = bf_lo(w[q]); e[2 * q + 1] = bf_hi(w[q]); }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4u v = ldnt(a.w, 4 * gb + q);
                e[4 * q] = as_f(v.x); e[4 * q + 1] = as_f(v.y); e[4 * q + 2] = as_f(v.z); e[4 * q + 3] = as_f(v.w);
            }
        }
        uint32_t m = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) m = umax(m, as_u(e[q]) & 0x7FFFFFFFu);
        const float amax_b = as_f(m);
        const uint32_t c_lo = block_scale_code<FAST>(amax_b * a.k_lo, s_g, rcp_g);
        const uint32_t c_hi = block_scale_code<FAST>(amax_b * a.k_hi, s_g, rcp_g);
        // Candidates from the largest code down; "<=" keeps the lowest code
        // among equal errors, which is the first candidate in k order.  A
        // candidate whose largest element alone already costs more than the
        // best error so far cannot win; once the largest element is clipped
        // (6 s <= amax_b) that cost only grows for smaller codes, so stop.
        // Each lane skips its own pruned candidates before every full
        // evaluation, so a wave runs as many evaluations as its busiest lane
        // needs, not one per candidate position any lane evaluates.
        uint32_t best = c_hi;
        float best_err = __builtin_inff();
        const int n = (int)(c_hi - c_lo) + 1;
        int j = 0;
        for (;;) {
            float sj = 0.0f, rj = 0.0f;
            bool done = false;
            for (;;) {
                if (j >= n) { done = true; break; }
                sj = tab.seff[c_hi - j];
                rj = tab.rcp[c_hi - j];
                if (!(max_term<FAST>(amax_b, sj, rj) > best_err)) break;
                if (6.0f * sj <= amax_b) { done = true; break; }
                ++j;
            }
            if (done) break;
            const float err = block_error<FAST>(e, sj, rj);
            if (err <= best_err) { best_err = err; best = c_hi - (uint32_t)j; }
            ++j;
        }
        a.scales_out[gb] = (uint8_t)best;
    }
}

template <bool BF16>
__global__ __launch_bounds__(kQThreads) void mse_kernel(MseArgs a, int64_t groups, int64_t P, const uint32_t* ws)
{
    __shared__ ScaleTable tab;
    const int64_t b = blockIdx.x / groups, g = blockIdx.x - b * groups;
    const float s_g = tensor_scale_of(ws[b * record_words(P)]);
    build_table(tab, s_g);
    if (g == 0 && threadIdx.x == 0) a.tscale_out[b] = s_g;
    __syncthreads();
    if (s_g >= kFastMinScale) calibrate_tensor<BF16, true>(a, b, g, groups, tab, s_g);
    else calibrate_tensor<BF16, false>(a, b, g, groups, tab, s_g);
}

// resident workgroups of a kernel on the current device (cached per device)
template <bool BF16, bool FP8>
int64_t resident_groups()
{
    static int64_t cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int64_t v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (v) return v;
    auto kernel = quantize_kernel<BF16, MODE_ONEPASS, FP8>;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kQThreads, 0) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    v = (int64_t)per_cu * cus;
    __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);
    return v;
}

} // namespace

int64_t quantize_chunks(bool bf16, int64_t elems)
{
    const int64_t units = elems >> 3;
    const int64_t per = bf16 ? Chunk<true>::UNITS : Chunk<false>::UNITS;
    return (units + per - 1) / per;
}

int64_t amax_chunks(int64_t bytes_per_tensor)
{
    const int64_t vecs = bytes_per_tensor / 16;
    const int64_t per = (int64_t)kQThreads * 8; // 32 KiB, as the quantizer's chunk
    return (vecs + per - 1) / per;
}

hipError_t launch_fill_u32(uint32_t* out, int64_t n, uint32_t v, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    int64_t grid = (n + kQThreads - 1) / kQThreads;
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)grid), dim3(kQThreads), 0, stream, out, n, v);
    return hipGetLastError();
}

hipError_t launch_copy_u32(const uint32_t* src, uint32_t* dst, int64_t n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    int64_t grid = (n + kQThreads - 1) / kQThreads;
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(copy_u32_kernel, dim3((unsigned)grid), dim3(kQThreads), 0, stream, src, dst, n);
    return hipGetLastError();
}

hipError_t launch_amax(const void* x, bool bf16, int64_t B, int64_t elems, uint32_t* ws, hipStream_t stream)
{
    const int64_t bytes = elems * (bf16 ? 2 : 4);
    const int64_t P = amax_chunks(bytes);
    if (B <= 0 || P <= 0) return hipSuccess;
    hipError_t e = launch_fill_u32(ws, B * record_words(P), 0u, stream);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(B * P));
    if (bf16) hipLaunchKernelGGL(amax_kernel<true>, grid, dim3(kQThreads), 0, stream, x, bytes / 16, P, ws);
    else hipLaunchKernelGGL(amax_kernel<false>, grid, dim3(kQThreads), 0, stream, x, bytes / 16, P, ws);
    return hipGetLastError();
}

hipError_t launch_amax_out(const uint32_t* ws, int64_t B, int64_t elems, bool bf16, uint32_t* out, hipStream_t stream)
{
    const int64_t P = amax_chunks(elems * (bf16 ? 2 : 4));
    if (B <= 0) return hipSuccess;
    if (P <= 0) return launch_fill_u32(out, B, 0u, stream);
    hipLaunchKernelGGL(amax_out_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, stream, ws, B, P, out);
    return hipGetLastError();
}

bool quantize_one_pass_ok(bool bf16, bool fp8, int64_t B, int64_t elems)
{
    const int64_t P = quantize_chunks(bf16, elems);
    const int64_t resident = fp8 ? (bf16 ? resident_groups<true, true>() : resident_groups<false, true>())
                                 : (bf16 ? resident_groups<true, false>() : resident_groups<false, false>());
    (void)B;
    return P >= 1 && resident > 0 && P <= resident / 2;
}

hipError_t launch_quantize(const QuantizeArgs& a, int mode, uint32_t* ws, hipStream_t stream)
{
    if (a.B <= 0 || a.elems <= 0) return hipSuccess;
    // the amax kernel and the quantizer cut a tensor into the same 32 KiB chunks
    const int64_t P = quantize_chunks(a.bf16, a.elems);
    if (mode == MODE_ONEPASS) {
        hipError_t e = launch_fill_u32(ws, a.B * record_words(P), 0u, stream);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)(a.B * P)), block(kQThreads);
#define QK(BF, M, F8) hipLaunchKernelGGL((quantize_kernel<BF, M, F8>), grid, block, 0, stream, a, P, ws)
#define QK2(M, F8) { if (a.bf16) QK(true, M, F8); else QK(false, M, F8); }
    if (mode == MODE_ONEPASS) {
        if (a.fp8) QK2(MODE_ONEPASS, true) else QK2(MODE_ONEPASS, false)
    } else if (mode == MODE_AMAX) {
        if (a.fp8) QK2(MODE_AMAX, true) else QK2(MODE_AMAX, false)
    } else {
        if (a.fp8) QK2(MODE_FROZEN, true) else QK2(MODE_FROZEN, false)
    }
#undef QK2
#undef QK
    return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream)
{
    const int64_t vecs = bytes / 16;
    const int tail_halves = (int)((bytes - vecs * 16) / 2);
    if (vecs == 0 && tail_halves == 0) return hipSuccess;
    int64_t grid = (vecs + kQThreads * 4 - 1) / (kQThreads * 4);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(kQThreads), 0, stream, src, dst, vecs,
                       (const uint16_t*)((const char*)src + vecs * 16), (uint16_t*)((char*)dst + vecs * 16),
                       tail_halves);
    return hipGetLastError();
}

int64_t clip_chunks(int64_t elems)
{
    const int64_t per = (int64_t)kQThreads * kClipUnits;
    return ((elems >> 3) + per - 1) / per;
}

hipError_t launch_qdq_bwd_clipped(const ClipArgs& a, hipStream_t stream)
{
    if (a.B <= 0 || a.elems <= 0) return hipSuccess;
    const int64_t P = clip_chunks(a.elems);
    const dim3 grid((unsigned)(a.B * P)), block(kQThreads);
#define CK(G, X) hipLaunchKernelGGL((clip_ste_kernel<G, X>), grid, block, 0, stream, a, P)
    if (a.gbf16) {
        if (a.xbf16) CK(true, true); else CK(true, false);
    } else {
        if (a.xbf16) CK(false, true); else CK(false, false);
    }
#undef CK
    return hipGetLastError();
}

hipError_t launch_sgd_step(const SgdArgs& a, hipStream_t stream)
{
    if (a.B <= 0 || a.elems <= 0) return hipSuccess;
    const int64_t P = clip_chunks(a.elems);
    const dim3 grid((unsigned)(a.B * P)), block(kQThreads);
#define SK(W, G) hipLaunchKernelGGL((sgd_step_kernel<W, G>), grid, block, 0, stream, a, P)
    if (a.wbf16) {
        if (a.gbf16) SK(true, true); else SK(true, false);
    } else {
        if (a.gbf16) SK(false, true); else SK(false, false);
    }
#undef SK
    return hipGetLastError();
}

hipError_t launch_mse_calibrate(const MseArgs& a, uint32_t* ws, hipStream_t stream)
{
    if (a.B <= 0 || a.elems <= 0) return hipSuccess;
    hipError_t e = launch_amax(a.w, a.bf16, a.B, a.elems, ws, stream);
    if (e != hipSuccess) return e;
    const int64_t P = amax_chunks(a.elems * (a.bf16 ? 2 : 4));
    const int64_t nblk = a.elems >> 4;
    int64_t groups = (nblk + kQThreads - 1) / kQThreads;
    const int64_t want = (16384 + a.B - 1) / a.B;
    if (groups > want) groups = want;
    if (groups < 1) groups = 1;
    const dim3 grid((unsigned)(groups * a.B));
    if (a.bf16) hipLaunchKernelGGL(mse_kernel<true>, grid, dim3(kQThreads), 0, stream, a, groups, P, ws);
    else hipLaunchKernelGGL(mse_kernel<false>, grid, dim3(kQThreads), 0, stream, a, groups, P, ws);
    return hipGetLastError();
}

} // namespace qad
