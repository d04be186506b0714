// Exhaustive check of the two gfx950 conversion instructions the NVFP4
// kernels use, against their reference definitions, on every binary32 input:
//  * v_cvt_scalef32_pk_fp4_f32 with unit scale: E2M1 code of x = nearest grid
//    value {0,.5,1,1.5,2,3,4,6} (midpoints go to the even code index), beyond
//    6 saturating, sign bit copied from x (NaN inputs skipped);
//  * v_cvt_scalef32_pk_f32_fp4 with unit scale: the 16 signed grid values;
//  * v_cvt_pk_bf16_f32: round to nearest even of the top 16 bits (NaNs
//    skipped), i.e. (u + 0x7FFF + ((u >> 16) & 1)) >> 16.
//  * v_cvt_scalef32_pk_fp8_f32 with unit scale: OCP E4M3FN code of x =
//    nearest magnitude of the format (ties to the even code), sign bit
//    copied, on every input up to 448 in magnitude; inputs beyond are
//    counted by what they give (the quantizer clamps its quotients to 448);
//  * v_cvt_scalef32_pk_f32_fp8 with unit scale: every non-NaN code decodes
//    to its value, in either half of the source word.
// Prints one line "fp4_mismatch bf16_mismatch decode_ok layout_word
// fp8_mismatch fp8_decode_ok fp8_layout_word".
// Built by the package build step; run by tests/test_gpu_cvt_instructions.py.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>

__device__ unsigned ref_e2m1(float r)
{
    const unsigned sign = __float_as_uint(r) >> 31;
    const float a = __builtin_fabsf(r);
    unsigned i;
    if (a <= 0.25f) i = 0;
    else if (a < 0.75f) i = 1;
    else if (a <= 1.25f) i = 2;
    else if (a < 1.75f) i = 3;
    else if (a <= 2.5f) i = 4;
    else if (a < 3.5f) i = 5;
    else if (a <= 5.0f) i = 6;
    else i = 7;
    return sign << 3 | i;
}

typedef short fp8x2_t __attribute__((ext_vector_type(2)));

// E4M3FN magnitude of code c (0..126): 4 exponent bits (bias 7), 3 mantissa
// bits, exponent 0 subnormal
__device__ float e4m3_mag(unsigned c)
{
    const unsigned e = c >> 3, m = c & 7;
    return e ? ldexpf(1.0f + m / 8.0f, (int)e - 7) : ldexpf((float)m, -9);
}

// nearest magnitude code, ties to the even code (the format's 127 values in
// order; binary search for the largest one <= a)
__device__ unsigned ref_e4m3(float a)
{
    unsigned lo = 0, hi = 126;
    while (lo < hi) {
        const unsigned mid = (lo + hi + 1) / 2;
        if (e4m3_mag(mid) <= a) lo = mid; else hi = mid - 1;
    }
    if (lo == 126u) return 126u;
    const float d0 = a - e4m3_mag(lo), d1 = e4m3_mag(lo + 1) - a;
    if (d0 < d1) return lo;
    if (d1 < d0) return lo + 1;
    return (lo & 1u) ? lo + 1 : lo;
}

__global__ void check_fp8(unsigned long long* bad)
{
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; // 2^24 threads x 256 inputs
    unsigned n = 0;
    for (unsigned k = 0; k < 256; ++k) {
        const unsigned u = (unsigned)(t * 256 + k);
        const float f = __uint_as_float(u), a = __builtin_fabsf(f);
        if (!(a <= 448.0f)) continue;   // NaN, or beyond the range the quantizer feeds
        fp8x2_t w = {0, 0};
        w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, f, -f, 1.0f, false);
        const unsigned ww = __builtin_bit_cast(unsigned, w), want = ref_e4m3(a);
        n += (ww & 0xFFu) != (((u >> 31) << 7) | want);
        n += ((ww >> 8) & 0xFFu) != ((((u >> 31) ^ 1u) << 7) | want);
        n += (ww >> 16) != 0u;
    }
    if (n) atomicAdd(bad + 2, (unsigned long long)n);
}

__global__ void check(unsigned long long* bad)
{
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; // 2^24 threads x 256 inputs
    unsigned nf = 0, nb = 0;
    for (unsigned k = 0; k < 256; k += 2) {
        const unsigned u0 = (unsigned)(t * 256 + k), u1 = u0 + 1;
        const float f0 = __uint_as_float(u0), f1 = __uint_as_float(u1);
        const bool n0 = (u0 & 0x7FFFFFFFu) > 0x7F800000u, n1 = (u1 & 0x7FFFFFFFu) > 0x7F800000u;
        const unsigned hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f0, f1, 1.0f, 0);
        if (!n0 && (hw & 0xFu) != ref_e2m1(f0)) nf++;
        if (!n1 && ((hw >> 4) & 0xFu) != ref_e2m1(f1)) nf++;
        const __bf16 b0 = (__bf16)f0, b1 = (__bf16)f1;
        const unsigned h0 = __builtin_bit_cast(uint16_t, b0), h1 = __builtin_bit_cast(uint16_t, b1);
        if (!n0 && h0 != ((u0 + 0x7FFFu + ((u0 >> 16) & 1u)) >> 16)) nb++;
        if (!n1 && h1 != ((u1 + 0x7FFFu + ((u1 >> 16) & 1u)) >> 16)) nb++;
    }
    if (nf) atomicAdd(bad, (unsigned long long)nf);
    if (nb) atomicAdd(bad + 1, (unsigned long long)nb);
}

__global__ void decode_and_layout(unsigned* out)
{
    const float grid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    unsigned ok = 1;
    for (unsigned c = 0; c < 16; ++c) {
        for (int sel = 0; sel < 4; ++sel) {
            const unsigned word = (c | (c << 4)) << (8 * sel);
            float lo, hi;
            switch (sel) {
            case 0: { auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0); lo = v[0]; hi = v[1]; break; }
            case 1: { auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1); lo = v[0]; hi = v[1]; break; }
            case 2: { auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2); lo = v[0]; hi = v[1]; break; }
            default: { auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3); lo = v[0]; hi = v[1]; break; }
            }
            const float want = (c & 8) ? -grid[c & 7] : grid[c & 7];
            ok &= __float_as_uint(lo) == __float_as_uint(want) && __float_as_uint(hi) == __float_as_uint(want);
        }
    }
    unsigned w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, 0.5f, 1.0f, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, 1.5f, 2.0f, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, 3.0f, 4.0f, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, 6.0f, -0.5f, 1.0f, 3);
    out[0] = ok;
    out[1] = w;
    unsigned ok8 = 1;
    for (unsigned c = 0; c < 256; ++c) {
        if ((c & 0x7Fu) == 0x7Fu) continue;   // NaN codes
        const float want = (c & 0x80u) ? -e4m3_mag(c & 0x7Fu) : e4m3_mag(c & 0x7Fu);
        const unsigned lo = c | (c << 8), hi = lo << 16;
        const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 1.0f, false);
        const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, true);
        ok8 &= __float_as_uint(a[0]) == __float_as_uint(want) && __float_as_uint(a[1]) == __float_as_uint(want);
        ok8 &= __float_as_uint(b[0]) == __float_as_uint(want) && __float_as_uint(b[1]) == __float_as_uint(want);
    }
    fp8x2_t v = {0, 0};
    v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, 1.0f, -2.0f, 1.0f, false);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v, 448.0f, 0.001953125f, 1.0f, true);
    out[2] = ok8;
    out[3] = __builtin_bit_cast(unsigned, v);
}

int main()
{
    unsigned long long* bad;
    unsigned* out;
    if (hipMalloc(&bad, 24) != hipSuccess || hipMalloc(&out, 16) != hipSuccess) return 2;
    if (hipMemset(bad, 0, 24) != hipSuccess) return 2;
    check<<<65536, 256>>>(bad);
    check_fp8<<<65536, 256>>>(bad);
    decode_and_layout<<<1, 1>>>(out);
    if (hipDeviceSynchronize() != hipSuccess) return 3;
    unsigned long long b[3];
    unsigned o[4];
    if (hipMemcpy(b, bad, 24, hipMemcpyDeviceToHost) != hipSuccess || hipMemcpy(o, out, 16, hipMemcpyDeviceToHost) != hipSuccess)
        return 3;
    printf("%llu %llu %u 0x%08x %llu %u 0x%08x\n", b[0], b[1], o[0], o[1], b[2], o[2], o[3]);
    return 0;
}
