// Exhaustive check of the two gfx950 conversion instructions the NVFP4
// kernels use, against their reference definitions, on every binary32 input:
//  * v_cvt_scalef32_pk_fp4_f32 with unit scale: E2M1 code of x = nearest grid
//    value {0,.5,1,1.5,2,3,4,6} (midpoints go to the even code index), beyond
//    6 saturating, sign bit copied from x (NaN inputs skipped);
//  * v_cvt_scalef32_pk_f32_fp4 with unit scale: the 16 signed grid values;
//  * v_cvt_pk_bf16_f32: round to nearest even of the top 16 bits (NaNs
//    skipped), i.e. (u + 0x7FFF + ((u >> 16) & 1)) >> 16.
// Prints one line "fp4_mismatch bf16_mismatch decode_ok layout_word".
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
}

int main()
{
    unsigned long long* bad;
    unsigned* out;
    if (hipMalloc(&bad, 16) != hipSuccess || hipMalloc(&out, 8) != hipSuccess) return 2;
    if (hipMemset(bad, 0, 16) != hipSuccess) return 2;
    check<<<65536, 256>>>(bad);
    decode_and_layout<<<1, 1>>>(out);
    if (hipDeviceSynchronize() != hipSuccess) return 3;
    unsigned long long b[2];
    unsigned o[2];
    if (hipMemcpy(b, bad, 16, hipMemcpyDeviceToHost) != hipSuccess || hipMemcpy(o, out, 8, hipMemcpyDeviceToHost) != hipSuccess)
        return 3;
    printf("%llu %llu %u 0x%08x\n", b[0], b[1], o[0], o[1]);
    return 0;
}
