/*
 * Check of the division scheme the HIP kernels use for x / s when one divisor
 * s serves many elements: y = RN(1/s) once, then per element
 *     q0 = RN(x*y); q1 = q0 + RN(x - s*q0)*y; q2 = q1 + RN(x - s*q1)*y
 * (each correction one fused multiply-add).  q1 is a faithful quotient, so
 * Markstein's theorem makes q2 the correctly rounded x/s wherever no
 * intermediate under- or overflows.  The kernels take this path only when the
 * tensor scale is >= 2^-80 (so s >= 2^-89) and need the exact quotient only
 * where it can change a code: E2M1 element codes need |x/s| in [1/16, 16],
 * the E4M3 block scale amax_b/6/s_g needs quotients in [2^-12, 2^10].  The
 * exact claim is checked over [2^-12, 2^10]; everywhere else only the E2M1
 * magnitude index must agree (a code's sign bit is taken from x, never from
 * the quotient).  The sweep:
 *   - every positive finite bf16 x (both signs) against each divisor,
 *   - binary32 x within +-64 ulps of every E2M1 rounding midpoint times s,
 *   - random binary32 x with |x/s| in [1/16, 16],
 *   - random binary32 x with |x/s| in [2^-12, 2^10],
 * for divisors: 6, every E4M3 value times assorted tensor scales, plus random
 * binary32 in [2^-89, 2^100].
 * The signed form the quantizer uses (residuals negated: e = s*q - x, then
 * q + e*(-y)) must equal copysign(quot(|x|), x) bit for bit on every input
 * above whose quotient does not overflow (x*y = inf turns both forms into
 * NaN; the quantizer never lets that happen: dynamic scales keep quotients
 * below 12 and frozen ones see x clamped to +-8 s first), and on +-0 for
 * every divisor and for s = 0 (y = 0).
 * Prints: exact-range-checked, exact-range-mismatches, code-mismatches,
 * signed-form-mismatches.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static const double GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
static unsigned nearest_code(float r)
{
    double a = fmin(fabs((double)r), 1048576.0);
    unsigned best = 0;
    double bd = INFINITY;
    for (unsigned i = 0; i < 8; ++i) {
        double d = fabs(a - GRID[i]);
        if (d < bd || (d == bd && (i % 2 == 0))) { bd = d; best = i; }
    }
    if (isnan(r) || isinf(r)) best = 7;
    return ((f2u(r) >> 31) << 3) | best;
}

static float quot(float x, float s, float y)
{
    float q0 = x * y;
    float r0 = fmaf(-s, q0, x);
    float q1 = fmaf(r0, y, q0);
    float r1 = fmaf(-s, q1, x);
    return fmaf(r1, y, q1);
}

static float quot_signed(float x, float s, float y)
{
    float q0 = x * y;
    float r0 = fmaf(s, q0, -x);
    float q1 = fmaf(r0, -y, q0);
    float r1 = fmaf(s, q1, -x);
    return fmaf(r1, -y, q1);
}

int main(void)
{
    enum { ND = 4000 };
    static float divs[ND];
    int nd = 0;
    divs[nd++] = 6.0f;
    float sg[] = {1.0f, 3.7e-5f, 0.0625f / 3.0f, 1.1920929e-7f, 123.456f, 8.6736174e-19f, 5.0e20f};
    for (unsigned t = 0; t < sizeof sg / sizeof sg[0]; ++t)
        for (unsigned c = 1; c < 0x7F; ++c) {
            unsigned e = c >> 3, m = c & 7;
            float d = e ? ldexpf(1.0f + m / 8.0f, (int)e - 7) : ldexpf((float)m, -9);
            float s = d * sg[t];
            if (s >= 0x1p-89f) divs[nd++] = s;
        }
    uint64_t st = 0x9E3779B97F4A7C15ull;
    while (nd < ND) {
        st ^= st << 13; st ^= st >> 7; st ^= st << 17;
        uint32_t ex = 127 - 89 + (uint32_t)(st % (89 + 100 + 1));
        st ^= st << 13; st ^= st >> 7; st ^= st << 17;
        divs[nd++] = u2f((ex << 23) | (uint32_t)(st & 0x7FFFFF));
    }
    const float MID[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    unsigned long long exact_checked = 0, exact_bad = 0, code_bad = 0, signed_bad = 0;
    /* zeros: every divisor, and a zero divisor with y = 0 */
    for (int i = 0; i <= ND; ++i) {
        float s = i < ND ? divs[i] : 0.0f, y = i < ND ? 1.0f / s : 0.0f;
        for (int sg = 0; sg < 2; ++sg) {
            float z = sg ? -0.0f : 0.0f;
            signed_bad += f2u(quot_signed(z, s, y)) != f2u(copysignf(quot(0.0f, s, y), z));
        }
        if (i == ND)
            for (uint32_t h = 1; h < 0x7F80; ++h) {
                float x = u2f(h << 16);
                signed_bad += f2u(quot_signed(x, 0.0f, 0.0f)) != f2u(0.0f);
                signed_bad += f2u(quot_signed(-x, 0.0f, 0.0f)) != f2u(-0.0f);
            }
    }
#pragma omp parallel for reduction(+ : exact_checked, exact_bad, code_bad, signed_bad) schedule(dynamic, 8)
    for (int i = 0; i < ND; ++i) {
        float s = divs[i], y = 1.0f / s;
        float xs[2];
        uint64_t loc = 0x12345678ull * (uint64_t)(i + 1);
#define CHECK(X)                                                                 \
        do {                                                                     \
            float x_ = (X), q_ = quot(x_, s, y), ref_ = x_ / s;                  \
            if (fabsf(ref_) >= 0x1p-12f && fabsf(ref_) <= 1024.0f) {             \
                exact_checked++;                                                 \
                exact_bad += f2u(q_) != f2u(ref_);                               \
            }                                                                    \
            code_bad += (nearest_code(q_) & 7) != (nearest_code(ref_) & 7);    \
            if (!isinf(x_ * y))                                                  \
                signed_bad += f2u(quot_signed(x_, s, y)) !=                      \
                              f2u(copysignf(quot(fabsf(x_), s, y), x_));         \
        } while (0)
        for (uint32_t h = 1; h < 0x7F80; ++h) {
            xs[0] = u2f(h << 16);
            CHECK(xs[0]);
            CHECK(-xs[0]);
        }
        for (int t = 0; t < 7; ++t) {
            float c = MID[t] * s;
            for (int k = -64; k <= 64; ++k) {
                float x = u2f((uint32_t)((int32_t)f2u(c) + k));
                CHECK(x);
                CHECK(-x);
            }
        }
        for (int k = 0; k < 20000; ++k) {
            loc ^= loc << 13; loc ^= loc >> 7; loc ^= loc << 17;
            float r = ldexpf(1.0f + (float)(loc & 0xFFFFFF) / 16777216.0f, (int)((loc >> 32) % 8) - 4);
            CHECK(r * s);
            loc ^= loc << 13; loc ^= loc >> 7; loc ^= loc << 17;
            r = ldexpf(1.0f + (float)(loc & 0xFFFFFF) / 16777216.0f, (int)((loc >> 32) % 22) - 12);
            CHECK(r * s);
        }
    }
    printf("%llu %llu %llu %llu\n", exact_checked, exact_bad, code_bad, signed_bad);
    return 0;
}
