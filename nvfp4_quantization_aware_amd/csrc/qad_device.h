// Device-side building blocks of libqad for gfx950: the E4M3 / E2M1 codecs
// written as bit manipulation on binary32 patterns, the shared-divisor
// correctly rounded division, and wave-level helpers.  Page legend and the
// numerical conventions are in include/libqad.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qad {

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// bf16 halves of a 32-bit word -> binary32 (exact widening)
__device__ __forceinline__ float bf_lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return as_f(w & 0xFFFF0000u); }

// Two binary32 values -> two bf16 (round to nearest even) packed in a word,
// `lo` in bits 0..15.  A two-lane vector conversion, so that it lowers to a
// single v_cvt_pk_bf16_f32 with both sources (converting the halves one by
// one costs two conversions, a shift and an or).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// IEEE 754-2019 maximum (a NaN operand gives NaN).  Unlike fmaxf it needs
// no quieting of its operands; gfx950 does it in v_maximum3_f32.
__device__ __forceinline__ float maxnan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// ---------------------------------------------------------------------------
// E4M3 (OCP E4M3FN) block scale, [Nano] "NVFP4-Format und warum es wichtig
// ist?".  Encode a non-negative binary32 value with round-to-nearest-even and
// saturation at 448 (code 0x7E).  Normal range: round the 23-bit mantissa to 3
// bits in the integer domain (a carry into the exponent is the correct
// result), then rebias 127 -> 7.  Below 2^-6: the value is m * 2^-9, so m is
// v * 512 (exact) rounded to nearest even; m == 8 is code 0x08 = 2^-6.
// The result is always a code in 0..0x7E (a NaN saturates, a negative value
// gives 0), so it can index a 128-entry table whatever the input.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float v)
{
    if (!(v <= 448.0f)) return 0x7Eu;
    if (!(v >= 0.015625f)) return (uint32_t)__builtin_rintf(__builtin_fmaxf(v, 0.0f) * 512.0f);
    const uint32_t u = as_u(v);
    const uint32_t t = u + 0x7FFFFu + ((u >> 20) & 1u);
    return (t >> 20) - (120u << 3);
}

__device__ __forceinline__ float e4m3_decode(uint32_t c)
{
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    return e ? as_f(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// ---------------------------------------------------------------------------
// x / s correctly rounded, with r = RN(1/s) precomputed once per divisor:
// q0 = RN(x r) is within two ulps; one correction q1 = q0 + RN(x - s q0) r is
// faithful; a second correction is then the correctly rounded quotient
// (Markstein's theorem).  Valid while nothing under- or overflows; callers
// use it only for s >= 2^-89 and need the exact value only where a code can
// depend on it.  r = 0 for s = 0 yields 0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float div_rcp(float x, float s, float r)
{
    const float q0 = x * r;
    const float e0 = __builtin_fmaf(-s, q0, x);
    const float q1 = __builtin_fmaf(e0, r, q0);
    const float e1 = __builtin_fmaf(-s, q1, x);
    return __builtin_fmaf(e1, r, q1);
}

// The same quotient with x's sign on every result, signed zeros included: the
// steps of div_rcp with each residual negated (s q - x, then multiplied by
// -r).  Negation is exact and rounding to nearest is symmetric, so every
// nonzero result equals div_rcp's, while a zero quotient (x = +-0, or r = 0
// for s = 0) keeps the sign of x instead of becoming +0.
__device__ __forceinline__ float div_rcp_signed(float x, float s, float r)
{
    const float q0 = x * r;
    const float e0 = __builtin_fmaf(s, q0, -x);
    const float q1 = __builtin_fmaf(e0, -r, q0);
    const float e1 = __builtin_fmaf(s, q1, -x);
    return __builtin_fmaf(e1, -r, q1);
}

// ---------------------------------------------------------------------------
// gfx950 FP4 conversions with unit scale.  Encoding rounds to the nearest
// E2M1 value with ties to the even code and saturates, taking the code's sign
// from the input's sign bit: checked equal to that definition on every
// non-NaN binary32 input.  SEL picks the byte of `word` receiving the pair
// (first value in the low nibble).  Decoding gives the exact signed grid
// values of the pair in byte SEL.
// ---------------------------------------------------------------------------
template <int SEL>
__device__ __forceinline__ uint32_t fp4_encode_pair(uint32_t word, float lo, float hi)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, lo, hi, 1.0f, SEL);
}

template <int SEL>
__device__ __forceinline__ void fp4_decode_pair(uint32_t word, float& lo, float& hi)
{
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
    lo = v[0];
    hi = v[1];
}

// swap with the neighbouring lane (lane ^ 1) through DPP quad_perm(1,0,3,2)
__device__ __forceinline__ uint32_t swap_pair(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// maximum over a wave of 64 lanes
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    for (int o = 32; o > 0; o >>= 1) v = umax(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

} // namespace qad
