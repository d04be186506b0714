// Fused KL(teacher || student) forward + backward over the vocabulary for
// gfx950 ([Nano] "Von QAT zu QAD": the student is trained to match the frozen
// teacher's output distribution; [Qwen] "3. QAD": logits are compared
// element-wise over the vocabulary and dense fp32 copies of them do not fit,
// so the loss streams bf16 logits and never materialises probabilities).
//
// One HBM pass.  A token row is cut into W segments, one workgroup each; a
// workgroup loads its segment once and keeps the packed logits in registers.
// Pass 1 reduces them to the segment's online-softmax state (max, sum of
// 2^(c x - m) for teacher and student, teacher-weighted sum of t - s; c =
// log2(e)/T, m the lane's own maxima).  The W states of a row are exchanged
// through the workspace and merged in segment order (so every workgroup of the
// row computes bit-identical row statistics, whatever the schedule).  Pass 2
// computes 2^(c x - m_row) / Z_row from the logits still in registers and
// writes the gradient (q - p) * grad_scale / T.  Recomputing two exponentials
// costs less than holding them: it keeps ~4 workgroups resident per CU,
// enough to hide the load and exchange latency.  Per-row losses go to row_loss; one
// workgroup sums them in a fixed order (binary64) for the mean.
#include "qad_device.h"
#include "qad_internal.h"

namespace qad {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 0x1.715476p+0f;  // RN(log2(e))
constexpr float kLn2 = 0x1.62e430p-1f;    // RN(ln(2))
// Segment shape: 256 lanes x 8 units of 8 logits = 16384 logits per tensor
// (64 KiB of bf16 teacher + student per workgroup; measured fastest among
// 64..1024 lanes x 2..24 units on MI355X).
#ifndef QAD_KL_THREADS
#define QAD_KL_THREADS 256
#endif
#ifndef QAD_KL_UNITS
#define QAD_KL_UNITS 8
#endif
constexpr int kSegThreads = QAD_KL_THREADS; // lanes per segment workgroup
constexpr int kSegUnits = QAD_KL_UNITS;     // 8-element units per lane, row and tensor
constexpr int64_t kSegSpan = (int64_t)kSegThreads * kSegUnits; // units per segment
constexpr int kMaxSegments = 64;           // longer rows take the two-pass kernel

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ v4u ldnt(const void* p, int64_t i) { return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p) + i); }
__device__ __forceinline__ void stnt(void* p, int64_t i, v4u v) { __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(p) + i); }

// A lane's (or a merged) online state: the running maxima m_t, m_s of c t
// and c s, the sums of 2^(c t - m_t) and 2^(c s - m_s), the teacher-weighted
// sum of t - s, and the largest s - t seen (which bounds the row's
// log-ratios log2(q/p) for pass 2).
struct Stats {
    float mt, zt, at, ms, zs, dx;
};

__device__ __forceinline__ Stats empty_stats()
{
    return Stats{-__builtin_inff(), 0.0f, 0.0f, -__builtin_inff(), 0.0f, -__builtin_inff()};
}

// merge two partial (max, sum) states; equal maxima (also both -inf) need no
// rescaling, which keeps empty partials from producing 0 * inf.  Symmetric in
// its operands, bit for bit.
__device__ __forceinline__ Stats merge(const Stats& a, const Stats& b)
{
    Stats r;
    r.mt = maxnan(a.mt, b.mt);
    const float fa = a.mt == r.mt ? 1.0f : exp2_hw(a.mt - r.mt);
    const float fb = b.mt == r.mt ? 1.0f : exp2_hw(b.mt - r.mt);
    r.zt = a.zt * fa + b.zt * fb;
    r.at = a.at * fa + b.at * fb;
    r.ms = maxnan(a.ms, b.ms);
    const float ga = a.ms == r.ms ? 1.0f : exp2_hw(a.ms - r.ms);
    const float gb = b.ms == r.ms ? 1.0f : exp2_hw(b.ms - r.ms);
    r.zs = a.zs * ga + b.zs * gb;
    r.dx = maxnan(a.dx, b.dx);
    return r;
}

__device__ __forceinline__ Stats shfl_xor_stats(const Stats& s, int o)
{
    return Stats{__shfl_xor(s.mt, o, 64), __shfl_xor(s.zt, o, 64), __shfl_xor(s.at, o, 64),
                 __shfl_xor(s.ms, o, 64), __shfl_xor(s.zs, o, 64), __shfl_xor(s.dx, o, 64)};
}

// workgroup reduction in a fixed order (xor tree in each wave, then waves in
// order); the result is returned to every lane
template <int NT>
__device__ Stats group_merge(Stats st, Stats* part)
{
    for (int o = 32; o > 0; o >>= 1) st = merge(st, shfl_xor_stats(st, o));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = st;
    __syncthreads();
    Stats r = part[0];
    for (int w = 1; w < NT / 64; ++w) r = merge(r, part[w]);
    __syncthreads();
    return r;
}

// per-lane sums of the term-wise KL (see termwise_kl)
struct LossAcc {
    float l, y, p;
};

// sums of the lanes' term-wise sums over the workgroup in binary64, fixed
// order; the result is returned to every lane
struct LossSum {
    double l, y, p;
};

template <int NT>
__device__ LossSum group_sum(const LossAcc& a, LossSum* part)
{
    LossSum v{(double)a.l, (double)a.y, (double)a.p};
    for (int o = 32; o > 0; o >>= 1) {
        v.l += __shfl_xor(v.l, o, 64);
        v.y += __shfl_xor(v.y, o, 64);
        v.p += __shfl_xor(v.p, o, 64);
    }
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    LossSum r = part[0];
    for (int w = 1; w < NT / 64; ++w) {
        r.l += part[w].l;
        r.y += part[w].y;
        r.p += part[w].p;
    }
    __syncthreads();
    return r;
}

template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t unit, bool valid, float (&v)[8])
{
    if constexpr (BF16) {
        const v4u w = valid ? ldnt(base, unit) : v4u{0u, 0u, 0u, 0u};
        v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
        v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
    } else {
        const v4u w0 = valid ? ldnt(base, 2 * unit) : v4u{0u, 0u, 0u, 0u};
        const v4u w1 = valid ? ldnt(base, 2 * unit + 1) : v4u{0u, 0u, 0u, 0u};
        v[0] = as_f(w0.x); v[1] = as_f(w0.y); v[2] = as_f(w0.z); v[3] = as_f(w0.w);
        v[4] = as_f(w1.x); v[5] = as_f(w1.y); v[6] = as_f(w1.z); v[7] = as_f(w1.w);
    }
}

__device__ __forceinline__ float max8(const float (&v)[8])
{
    return maxnan(maxnan(maxnan(v[0], v[1]), maxnan(v[2], v[3])), maxnan(maxnan(v[4], v[5]), maxnan(v[6], v[7])));
}

__device__ __forceinline__ float sum8(const float (&v)[8])
{
    return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

__device__ __forceinline__ void unpack8(v4u w, float (&v)[8])
{
    v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
    v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
}

// ---------------------------------------------------------------------------
// What a row's pass 2 needs, computed once per row (in binary64) from the
// merged statistics, and the row's loss by the difference form
//   KL = E_p[t - s]/T - (LSE_t - LSE_s),  LSE in log2 units m + log2 Z.
// That form subtracts two terms that are large next to a small KL (a student
// close to the teacher, or shifted from it by a constant): its binary32
// exponentials leave ~1e-7 nats of error.  Where the KL is not large against
// that (below 1/16 nat plus 1/16 of the two terms' magnitudes), the row's loss
// is taken instead in pass 2, element by element, in the form
//   KL = sum_v p_v psi(x_v),  x_v = log2(q_v / p_v),  psi(x) = 2^x - 1 - x ln 2,
// whose terms are all non-negative (the sum of p_v (2^x_v - 1) is sum q - sum p
// = 0), so it keeps its relative accuracy however small the KL, and whose
// first-order sensitivity to an error in the row's LSE difference is zero.
// ---------------------------------------------------------------------------
constexpr double kLn2d = 0.69314718055994530942;
constexpr double kRobustAbs = 1.0 / 16.0;   // nats
constexpr double kRobustRel = 1.0 / 16.0;

// Pass 2 takes one of three forms per row (the same in every workgroup of the
// row, all of which hold bit-identical statistics):
//   FORM_PLAIN  g = (P 2^x - P) 2^-40 with P = p grad_scale / T 2^40 and x =
//               log2(q/p) from s - t: one exponential of the teacher's logit
//               (the weight folded into its reference) and one of x; taken on
//               rows whose largest x is at most 14, so that q <= 2^14 p and P
//               stays a normal number wherever q is not negligible;
//   FORM_SELECT g = +-big (1 - 2^-|x|) from the larger of p and q: any x;
//   FORM_LOSS   FORM_SELECT, plus the row's KL term by term (rows whose KL
//               is small next to the difference form's rounding).
// The exponentials run above the row's references (2^kShift in the select
// forms, 2^40 in the plain one) so that probabilities far below the largest
// stay normal binary32 numbers (the hardware exponential flushes subnormal
// results); the weights carry the compensating powers of two.  A shifted
// reference may round: that scales every p (or q) of the row by the same
// factor within 2^-20, a relative error of the gradient well inside its band,
// and one the term-wise KL cancels (see termwise_kl).
constexpr float kShift = 32.0f;
constexpr double kPlainShift = 40.0;
constexpr double kPlainMaxX = 14.0;      // FORM_PLAIN's bound on x (a margin below 16)
enum { FORM_PLAIN = 0, FORM_SELECT = 1, FORM_LOSS = 2 };

struct RowConst {
    float mt, ms;      // select forms: row references of c t and c s, minus kShift
    float dh;          // x = log2(q / p) = c (s - t) - dh
    float wt, ws;      // grad_scale / T / Z_t and / Z_s, times 2^-kShift
    float izt, izs;    // 1 / Z_t and 1 / Z_s, times 2^-kShift
    float mtp;         // plain form: reference of c t giving p |grad_scale / T| 2^40
    float psc;         // plain form: 2^-40 with the sign of grad_scale
    float loss;        // the row's KL by the difference form
    uint32_t form;
};

// log2 of a positive binary32 value as its exponent plus log2 of its
// significand in [1, 2) (the hardware logarithm on a value near 1, so the
// result's absolute error stays near 1e-7 whatever the magnitude)
__device__ __forceinline__ double log2_split(float v)
{
    int e = 0;
    const float m = __builtin_frexpf(v, &e);   // v = m 2^e, m in [0.5, 1)
    return (double)(e - 1) + (double)__builtin_amdgcn_logf(2.0f * m);
}

// (one lane per workgroup; lgmul = log2 |grad_scale / T|)
__device__ __forceinline__ RowConst row_const(const Stats& st, float c, float inv_t, float gmul, float lgmul,
                                              bool want_grad)
{
    RowConst k;
    const float izt = __builtin_amdgcn_rcpf(st.zt), izs = __builtin_amdgcn_rcpf(st.zs);
    // log2 Z_t and log2 (Z_t / Z_s) (the quotient correctly rounded: equal sums give exactly 0)
    const double lt = log2_split(st.zt), lr = log2_split(st.zt / st.zs);
    const double t1 = (double)(st.at * izt) * (double)inv_t;
    const double t2 = kLn2d * (((double)st.mt - (double)st.ms) + lr);
    const double kl = t1 - t2;
    const double dh = ((double)st.ms - (double)st.mt) - lr;
    constexpr float kUnshift = 0x1p-32f;   // 2^-kShift
    k.mt = st.mt - kShift;
    k.ms = st.ms - kShift;
    k.dh = (float)dh;
    k.wt = gmul * izt * kUnshift;
    k.ws = gmul * izs * kUnshift;
    k.izt = izt * kUnshift;
    k.izs = izs * kUnshift;
    k.mtp = (float)((double)st.mt - kPlainShift - ((double)lgmul - lt));
    k.psc = gmul < 0.0f ? -0x1p-40f : 0x1p-40f;
    k.loss = (float)kl;
    const bool robust = !(kl >= kRobustAbs + kRobustRel * (__builtin_fabs(t1) + __builtin_fabs(t2)));
    // largest log2(q/p) of the row: c max(s - t) - dh
    const bool bounded = (double)c * (double)st.dx - dh <= kPlainMaxX;
    k.form = robust ? FORM_LOSS : (bounded || !want_grad) ? FORM_PLAIN : FORM_SELECT;
    return k;
}

// The term-wise KL of a row from three sums over its entries, with p' the
// probabilities as computed and x' the log-ratios as computed:
//   L = sum p' psi(x'),  Y = sum p' x' ln 2,  P = sum p'.
// If p' = p (1 + e_p) and x' = x + e for row constants e_p, e (the rounding
// of Z_t and of the row's offset dh), then D = L + Y = P (2^e - 1) and
//   KL = (L - (D - P log1p(D / P))) / P
// exactly: the constant errors cancel to every order (alone, L would carry
// e^2 ln^2(2) / 2, ~1e-14 nats, which is all of a KL near 1e-10).
__host__ __device__ inline double termwise_kl(double L, double Y, double P)
{
    const double D = L + Y;
    return (L - (D - P * log1p(D / P))) / P;
}

// Taylor coefficients of (e^y - 1 - y) / y^2 = 1/2! + y/3! + ... + y^6/8!
// (binary32; for |y| <= 1/2 the truncation is below 6e-8 of the sum)
constexpr float kPsi0 = 0.5f, kPsi1 = 1.0f / 6.0f, kPsi2 = 1.0f / 24.0f, kPsi3 = 1.0f / 120.0f,
                kPsi4 = 1.0f / 720.0f, kPsi5 = 1.0f / 5040.0f, kPsi6 = 1.0f / 40320.0f;

// Gradient of one logit pair, (q - p) grad_scale / T, from the larger of p and
// q and the ratio r = 2^-|x| of the smaller to it:
//   x >= 0 (q >= p):  q (1 - r) grad_scale / T,   q = 2^(c s - m_s) / Z_s
//   x <  0 (p >  q): -p (1 - r) grad_scale / T,   p = 2^(c t - m_t) / Z_t.
// Unlike the difference of the two separately rounded probabilities, this
// keeps its relative accuracy where q and p nearly agree (x is computed from
// s - t, not from two large exponents), and its rounding errors scale with
// |q - p|.  FORM_LOSS: also adds p psi(x) to acc (the term-wise KL, nats).
template <int FORM>
__device__ __forceinline__ float grad_elem(float t, float s, float c, const RowConst& k, LossAcc& acc)
{
    if constexpr (FORM == FORM_PLAIN) {
        const float E = exp2_hw(__builtin_fmaf(s - t, c, -k.dh));   // q / p
        const float P = exp2_hw(__builtin_fmaf(t, c, -k.mtp));      // p |grad_scale / T| 2^40
        return __builtin_fmaf(P, E, -P) * k.psc;
    }
    constexpr bool LOSS = FORM == FORM_LOSS;
    const float x = __builtin_fmaf(s - t, c, -k.dh);
    const bool pos = x >= 0.0f;
    const float v = pos ? s : t, m = pos ? k.ms : k.mt;
    const float a = __builtin_fmaf(v, c, -m);
    float big = exp2_hw(a);
    if constexpr (LOSS) {
        // the exponent c v - m is exact in binary64; its remainder after the
        // binary32 rounding a corrects 2^a to first order, so that p and q
        // hold their relative accuracy however far below the row's maximum
        // they are
        const double ad = (double)v * (double)c - (double)m;
        const float lo = (float)(ad - (double)a);
        big = __builtin_fmaf(big, lo * kLn2, big);
    }
    const float r = exp2_hw(-__builtin_fabsf(x));
    const float h = __builtin_fmaf(-big, r, big);
    const float g = h * (pos ? k.ws : -k.wt);
    if constexpr (LOSS) {
        // p psi(x): as q ((1 - r) - r y) or p ((r - 1) - y) with y = x ln 2,
        // and for |y| <= 1/2, where those cancel, as p y^2 P(y)
        const float y = x * kLn2;
        const float pm = big * (pos ? k.izs : k.izt);   // max(p, q)
        const float pp = pos ? pm * r : pm;             // p
        const float om = 1.0f - r;
        const float dir = pos ? __builtin_fmaf(-r, y, om) : -om - y;
        float P = __builtin_fmaf(kPsi6, y, kPsi5);
        P = __builtin_fmaf(P, y, kPsi4);
        P = __builtin_fmaf(P, y, kPsi3);
        P = __builtin_fmaf(P, y, kPsi2);
        P = __builtin_fmaf(P, y, kPsi1);
        P = __builtin_fmaf(P, y, kPsi0);
        const float sm = (y * y) * P * (pos ? r : 1.0f);
        acc.l = __builtin_fmaf(pm, __builtin_fabsf(y) <= 0.5f ? sm : dir, acc.l);
        acc.y = __builtin_fmaf(pp, y, acc.y);
        acc.p += pp;
    }
    return g;
}

// One unit of 8 teacher and 8 student logits, as held in registers: one
// 16-byte vector per tensor for bf16, two for fp32.
template <bool BF16>
struct Unit {
    static constexpr int V = BF16 ? 1 : 2;
    v4u t[V], s[V];

    __device__ void load(const KlArgs& a, int64_t unit, bool valid)
    {
#pragma unroll
        for (int q = 0; q < V; ++q) {
            t[q] = valid ? ldnt(a.teacher, V * unit + q) : v4u{0u, 0u, 0u, 0u};
            s[q] = valid ? ldnt(a.student, V * unit + q) : v4u{0u, 0u, 0u, 0u};
        }
    }
    __device__ void values(float (&tv)[8], float (&sv)[8]) const
    {
        if constexpr (BF16) {
            unpack8(t[0], tv);
            unpack8(s[0], sv);
        } else {
            tv[0] = as_f(t[0].x); tv[1] = as_f(t[0].y); tv[2] = as_f(t[0].z); tv[3] = as_f(t[0].w);
            tv[4] = as_f(t[1].x); tv[5] = as_f(t[1].y); tv[6] = as_f(t[1].z); tv[7] = as_f(t[1].w);
            sv[0] = as_f(s[0].x); sv[1] = as_f(s[0].y); sv[2] = as_f(s[0].z); sv[3] = as_f(s[0].w);
            sv[4] = as_f(s[1].x); sv[5] = as_f(s[1].y); sv[6] = as_f(s[1].z); sv[7] = as_f(s[1].w);
        }
    }
};

// Gradients of one unit (masked by the teacher threshold when TOPK) as the
// words unit_grad stores: bf16 in lo (GRAD 1), or binary32 in lo and hi
// (GRAD 2); LOSS adds the unit's term-wise KL to acc.
template <int GRAD, bool TOPK, int FORM>
__device__ __forceinline__ void unit_grad_words(const float (&tv)[8], const float (&sv)[8], float c, float tau,
                                                const RowConst& k, LossAcc& acc, v4u& lo, v4u& hi)
{
    float g[8];
    LossAcc ua{0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        LossAcc e{0.0f, 0.0f, 0.0f};
        g[i] = grad_elem<FORM>(tv[i], sv[i], c, k, e);
        if (TOPK && !(tv[i] >= tau)) { g[i] = 0.0f; e = LossAcc{0.0f, 0.0f, 0.0f}; }
        ua.l += e.l;
        ua.y += e.y;
        ua.p += e.p;
    }
    if (FORM == FORM_LOSS) {
        acc.l += ua.l;
        acc.y += ua.y;
        acc.p += ua.p;
    }
    if constexpr (GRAD == 1) {
        lo = v4u{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]), pack_bf16x2(g[6], g[7])};
    } else if constexpr (GRAD == 2) {
        lo = v4u{as_u(g[0]), as_u(g[1]), as_u(g[2]), as_u(g[3])};
        hi = v4u{as_u(g[4]), as_u(g[5]), as_u(g[6]), as_u(g[7])};
    }
}

// the words of unit_grad_words written to `unit` of the gradient
template <int GRAD>
__device__ __forceinline__ void store_grad_unit(const KlArgs& a, int64_t unit, v4u lo, v4u hi)
{
    if constexpr (GRAD == 1) {
        stnt(a.grad, unit, lo);
    } else if constexpr (GRAD == 2) {
        stnt(a.grad, 2 * unit, lo);
        stnt(a.grad, 2 * unit + 1, hi);
    }
}

template <int GRAD, bool TOPK, int FORM>
__device__ __forceinline__ void unit_grad(const float (&tv)[8], const float (&sv)[8], float c, float tau,
                                          const RowConst& k, const KlArgs& a, int64_t unit, LossAcc& acc)
{
    v4u lo{0u, 0u, 0u, 0u}, hi{0u, 0u, 0u, 0u};
    unit_grad_words<GRAD, TOPK, FORM>(tv, sv, c, tau, k, acc, lo, hi);
    store_grad_unit<GRAD>(a, unit, lo, hi);
}

// Opaque to the optimiser: values derived from v before this point cannot be
// reused after it.  Used so that widened logits are recomputed from the packed
// registers where needed instead of being kept alive (64 extra registers).
__device__ __forceinline__ void refresh(v4u& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ int64_t lane_unit(int64_t seg_u0, int k) { return seg_u0 + k * kSegThreads + threadIdx.x; }

// A lane's state over its units of one segment, in one pass: unit by unit
// in ascending order, the running maxima (of c x) are raised to the unit's
// and the sums of 2^(c x - m) and the teacher-weighted sum of t - s are
// rescaled by 2^(m_old - m_new) when they move, then the unit is added.  A
// unit is thus consumed as soon as its loads land, while later units are
// still in flight.  `get(k, unit)` supplies unit k: from registers in the
// segment's own workgroup (UNROLL), from memory one unit at a time in the
// bounded wait's fallback.  FULL: every unit lies inside the row.  The
// arithmetic is the same in every form (a unit past the row end is skipped
// and a valid one takes the same operations), so all give bit-identical
// states.
template <bool BF16, bool UNROLL, bool FULL, bool TOPK, class Get>
__device__ __forceinline__ Stats lane_state(int64_t seg_u0, int64_t units, float c, float tau, Get get,
                                            uint32_t* kept_units = nullptr)
{
    constexpr int kUnroll = UNROLL ? kSegUnits : 1;
    float mt = -__builtin_inff(), ms = -__builtin_inff();
    float zt = 0.0f, zs = 0.0f, at = 0.0f, dx = -__builtin_inff();
#pragma unroll kUnroll
    for (int k = 0; k < kSegUnits; ++k) {
        const bool valid = FULL || lane_unit(seg_u0, k) < units;
        Unit<BF16> u;
        get(k, u);
        if (!valid) continue;
        float tv[8], sv[8], pt[8], ps[8];
        u.values(tv, sv);
        // TOPK: dropped entries become -inf, whose weights 2^(-inf) are
        // exactly 0 once a kept entry has set the maxima; a unit of this lane
        // with no kept entry changes nothing and is skipped (which also
        // keeps -inf - (-inf) out of the exponent).  dx takes every entry of
        // the units it sees, dropped ones too: it only has to bound the kept
        // entries' s - t from above (for the choice of pass 2's form), and a
        // maximum over more entries does, one select per entry cheaper.
        float d[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = tv[i] - sv[i];
        dx = maxnan(maxnan(maxnan(dx, -d[0]), maxnan(-d[1], -d[2])), maxnan(maxnan(-d[3], -d[4]), -d[5]));
        dx = maxnan(dx, maxnan(-d[6], -d[7]));
        if constexpr (TOPK) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool kept = tv[i] >= tau;
                tv[i] = kept ? tv[i] : -__builtin_inff();
                sv[i] = kept ? sv[i] : -__builtin_inff();
            }
        }
        const float tmax = max8(tv);
        if (TOPK && tmax == -__builtin_inff()) continue;
        if (TOPK && kept_units) *kept_units |= 1u << k;   // unit k holds a kept entry
        // c > 0: the max of the scaled logits is the scaled max
        const float nmt = maxnan(mt, tmax * c);
        const float nms = maxnan(ms, max8(sv) * c);
        // equal maxima (also both -inf) need no rescaling
        const float ft = nmt == mt ? 1.0f : exp2_hw(mt - nmt);
        const float fs = nms == ms ? 1.0f : exp2_hw(ms - nms);
        mt = nmt;
        ms = nms;
        float pa = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pt[i] = exp2_hw(__builtin_fmaf(tv[i], c, -mt));
            ps[i] = exp2_hw(__builtin_fmaf(sv[i], c, -ms));
            pa = __builtin_fmaf(pt[i], d[i], pa);
        }
        zt = zt * ft + sum8(pt);
        at = at * ft + pa;
        zs = zs * fs + sum8(ps);
        // unit by unit: later units' work is not hoisted above this point
        if (UNROLL) asm volatile("" : "+v"(zt), "+v"(zs), "+v"(at), "+v"(mt), "+v"(ms), "+v"(dx));
    }
    return Stats{mt, zt, at, ms, zs, dx};
}

// every lane's state over a segment held in registers
template <bool BF16, bool FULL, bool TOPK, class Regs>
__device__ __forceinline__ Stats lane_state_regs(Regs& m, int64_t seg_u0, int64_t units, float c, float tau,
                                                 uint32_t* kept_units)
{
    return lane_state<BF16, true, FULL, TOPK>(seg_u0, units, c, tau, [&](int k, Unit<BF16>& u) { u = m[k]; },
                                              kept_units);
}

// ---------------------------------------------------------------------------
// Per-row record of the segment kernels (rec_words(W) words, whole 128-byte
// lines, zeroed before each launch):
//   [0, 12 W)     segment s publishes its 6 state words (Stats) at 6 s .. 6 s + 5,
//                 each as a 64-bit {value, tag = 1} pair written by one
//                 single-copy-atomic store (no round trip for the writer); a
//                 reader waits until all 6 W tags are set;
//   [12 W, 18 W)  segment s's shares of the term-wise KL's three sums
//                 (binary64 L, Y, P), written after pass 2 on rows that take
//                 that form;
//   [18 W]        1 when the row takes the term-wise form (the mean kernel
//                 then adds the shares up and forms the row's loss);
//   [18 W + 1 + s] claim of segment s's state by a workgroup whose wait timed
//                 out (it then computes and publishes that state itself).
// ---------------------------------------------------------------------------
constexpr int kStateWords = 6;
__host__ __device__ inline int64_t rec_words(int W) { return (19 * (int64_t)W + 1 + 31) & ~(int64_t)31; }
__host__ __device__ inline int64_t share_word(int W, int seg) { return 12 * (int64_t)W + 6 * seg; }
__host__ __device__ inline int64_t flag_word(int W) { return 18 * (int64_t)W; }
__host__ __device__ inline int64_t claim_word(int W, int seg) { return 18 * (int64_t)W + 1 + seg; }

__device__ __forceinline__ float state_word(const Stats& st, int j)
{
    return j == 0 ? st.mt : j == 1 ? st.zt : j == 2 ? st.at : j == 3 ? st.ms : j == 4 ? st.zs : st.dx;
}

__device__ __forceinline__ Stats state_of_words(const uint32_t* w)
{
    return Stats{as_f(w[0]), as_f(w[1]), as_f(w[2]), as_f(w[3]), as_f(w[4]), as_f(w[5])};
}

__device__ __forceinline__ void publish(uint64_t* rec64, int seg, const Stats& st)
{
    const int tid = threadIdx.x;
    if (tid < kStateWords)
        __hip_atomic_store(rec64 + kStateWords * seg + tid, ((uint64_t)1 << 32) | as_u(state_word(st, tid)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0 waits (bounded) for all W segment states of a row and copies their
// words to `words` as they arrive; returns, to every lane of the workgroup,
// whether they all arrived.
__device__ __forceinline__ bool collect(const uint64_t* rec64, int W, uint32_t* words, uint32_t* flag,
                                        uint64_t wait_ticks)
{
    const int tid = threadIdx.x;
    if (tid < 64) {
        // lane l watches words l, l + 64, ... (6 W <= 6 kMaxSegments)
        constexpr int kPer = (kStateWords * kMaxSegments + 63) / 64;
        const int n = kStateWords * W;
        uint32_t got = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) got |= (tid + 64 * j >= n ? 1u : 0u) << j;
        const uint32_t all = (1u << kPer) - 1u;
        const uint64_t t0 = wall_clock64();
        bool done = false;
        while (true) {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = tid + 64 * j;
                if (!(got >> j & 1u)) {
                    const uint64_t w = __hip_atomic_load(rec64 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (w >> 32) {
                        words[i] = (uint32_t)w;
                        got |= 1u << j;
                    }
                }
            }
            done = __all(got == all);
            if (done) break;
            __builtin_amdgcn_s_sleep(2);
            if (wall_clock64() - t0 > wait_ticks) break;
        }
        if (tid == 0) *flag = done ? 1u : 0u;
    }
    __syncthreads();
    return *flag != 0u;  // the caller synchronises before the flag is written again
}

// Merge the W segment states of a row in a fixed tree (lane l of every wave
// starts from segment l; xor partners, merge is symmetric in its operands),
// so every workgroup of the row obtains bit-identical row statistics.
__device__ __forceinline__ Stats merge_segments(const uint32_t* words, int W)
{
    const int l = threadIdx.x & 63;
    Stats st = l < W ? state_of_words(words + kStateWords * l) : empty_stats();
    for (int o = 1; o < W; o <<= 1) st = merge(st, shfl_xor_stats(st, o));
    return Stats{__shfl(st.mt, 0, 64), __shfl(st.zt, 0, 64), __shfl(st.at, 0, 64), __shfl(st.ms, 0, 64),
                 __shfl(st.zs, 0, 64), __shfl(st.dx, 0, 64)};
}

template <bool BF16_IN>
using SegRegs = Unit<BF16_IN>[kSegUnits];

// issue the loads of one segment (units past the row end read as zeros)
template <bool BF16_IN, bool FULL>
__device__ __forceinline__ void seg_load(SegRegs<BF16_IN>& m, const KlArgs& a, int64_t row_unit0, int64_t seg_u0,
                                         int64_t units)
{
#pragma unroll
    for (int k = 0; k < kSegUnits; ++k)
        m[k].load(a, row_unit0 + lane_unit(seg_u0, k), FULL || lane_unit(seg_u0, k) < units);
}

// pass 1: the segment's state, identical in every lane
template <bool BF16_IN, bool FULL, bool TOPK>
__device__ __forceinline__ Stats seg_pass1(SegRegs<BF16_IN>& m, int64_t seg_u0, int64_t units, float c, float tau,
                                           Stats* part, uint32_t* kept_units)
{
    const Stats lane_st = lane_state_regs<BF16_IN, FULL, TOPK>(m, seg_u0, units, c, tau, kept_units);
    const Stats st = group_merge<kSegThreads>(lane_st, part);
#pragma unroll
    for (int k = 0; k < kSegUnits; ++k)
#pragma unroll
        for (int q = 0; q < Unit<BF16_IN>::V; ++q) { refresh(m[k].t[q]); refresh(m[k].s[q]); }
    return st;
}

struct SegShared {
    Stats part[kSegThreads / 64];
    LossSum lpart[kSegThreads / 64];
    uint32_t seg_words[kStateWords * kMaxSegments];
    RowConst rk;
    uint32_t flag;
};

// pass 2 over the units held in registers: the gradient, and in FORM_LOSS the
// lane's share of the term-wise KL
// Teacher-masked pass 2 on bf16 logits: most units of a top-k row hold no
// kept entry (k = 4096 of 131072: about 22% of 8-entry units hold one), and
// their gradient is all zeros.  A wave packs its units that hold a kept entry
// into LDS (up to kCompactUnits), its lanes take the packed units in turn, so
// the exponentials run for a few rounds of 64 units instead of all 8 per
// lane, and each result goes back through LDS to the unit's own lane, which
// stores its 8 units as the plain loop does (one coalesced 16-byte store per
// unit and lane; scattered stores from the packed order fragment the
// gradient's lines).  Each unit's arithmetic is unit_grad's, so the bits are
// those of the plain loop.  A wave with more such units than fit takes the
// plain loop.  Returns false then.
constexpr int kCompactUnits = 192;   // per wave: three rounds of 64
struct CompactUnits {
    v4u t[kSegThreads / 64][kCompactUnits];   // teacher words, then the gradient's low words
    v4u s[kSegThreads / 64][kCompactUnits];   // student words, then (binary32) its high words
};

// one buffer per kernel, whichever instances of the pass use it
__device__ __forceinline__ CompactUnits& compact_units()
{
    __shared__ CompactUnits cu;
    return cu;
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int GRAD, bool FULL, int FORM>
__device__ __forceinline__ bool seg_pass2_compact(SegRegs<true>& m, const KlArgs& a, int64_t row_unit0,
                                                  int64_t seg_u0, int64_t units, float c, float tau, const RowConst& k,
                                                  uint32_t kept_units)
{
    CompactUnits& cu = compact_units();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t n = (uint32_t)__builtin_popcount(kept_units);
    uint32_t incl = n;   // inclusive prefix sum over the wave's lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = (uint32_t)__shfl_up((int)incl, o, 64);
        if (lane >= o) incl += v;
    }
    const uint32_t total = (uint32_t)__shfl((int)incl, 63, 64);
    if (total > (uint32_t)kCompactUnits) return false;   // the same in every lane of the wave
    const uint32_t first = incl - n;
    uint32_t pos = first;
#pragma unroll
    for (int j = 0; j < kSegUnits; ++j) {
        if ((kept_units >> j) & 1u) {   // only valid units are marked
            cu.t[wave][pos] = m[j].t[0];
            cu.s[wave][pos] = m[j].s[0];
            ++pos;
        }
    }
    wave_lds_sync();
    LossAcc acc{0.0f, 0.0f, 0.0f};
    for (uint32_t r = (uint32_t)lane; r < total; r += 64) {
        Unit<true> u;
        u.t[0] = cu.t[wave][r];
        u.s[0] = cu.s[wave][r];
        float tv[8], sv[8];
        u.values(tv, sv);
        v4u lo{0u, 0u, 0u, 0u}, hi{0u, 0u, 0u, 0u};
        unit_grad_words<GRAD, true, FORM>(tv, sv, c, tau, k, acc, lo, hi);
        cu.t[wave][r] = lo;   // each slot is read and rewritten by one lane only
        if constexpr (GRAD == 2) cu.s[wave][r] = hi;
    }
    wave_lds_sync();
    pos = first;
#pragma unroll
    for (int j = 0; j < kSegUnits; ++j) {
        if (!FULL && lane_unit(seg_u0, j) >= units) continue;
        v4u lo{0u, 0u, 0u, 0u}, hi{0u, 0u, 0u, 0u};
        if ((kept_units >> j) & 1u) {
            lo = cu.t[wave][pos];
            if constexpr (GRAD == 2) hi = cu.s[wave][pos];
            ++pos;
        }
        store_grad_unit<GRAD>(a, row_unit0 + lane_unit(seg_u0, j), lo, hi);
    }
    return true;
}

template <bool BF16_IN, int GRAD, bool FULL, bool TOPK, int FORM>
__device__ __forceinline__ LossAcc seg_pass2(SegRegs<BF16_IN>& m, const KlArgs& a, int64_t row_unit0, int64_t seg_u0,
                                             int64_t units, float c, float tau, const RowConst& k,
                                             uint32_t kept_units)
{
    if constexpr (TOPK && BF16_IN && GRAD != 0 && FORM != FORM_LOSS) {
        if (seg_pass2_compact<GRAD, FULL, FORM>(m, a, row_unit0, seg_u0, units, c, tau, k, kept_units))
            return LossAcc{0.0f, 0.0f, 0.0f};
    }
    LossAcc acc{0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < kSegUnits; ++j) {
        if (!FULL && lane_unit(seg_u0, j) >= units) continue;
        float tv[8], sv[8];
        m[j].values(tv, sv);
        unit_grad<GRAD, TOPK, FORM>(tv, sv, c, tau, k, a, row_unit0 + lane_unit(seg_u0, j), acc);
    }
    return acc;
}

// the row's statistics (exchange + merge), its loss and pass 2 from the
// logits still held in registers
template <bool BF16_IN, int GRAD, bool FULL, bool TOPK>
__device__ __forceinline__ void seg_finish(SegRegs<BF16_IN>& m, const KlArgs& a, int W, int64_t row, int seg,
                                           const Stats& my_seg, float c, float tau, float gmul,
                                           uint32_t* rec_base, SegShared& sh, uint32_t kept_units)
{
    const int64_t units = a.vocab >> 3;
    const int64_t row_unit0 = row * units;
    const int64_t seg_u0 = seg * kSegSpan;
    uint32_t* rec = rec_base + row * rec_words(W);
    Stats row_st = my_seg;
    if (W > 1) {
        uint64_t* rec64 = reinterpret_cast<uint64_t*>(rec);
        if (!collect(rec64, W, sh.seg_words, &sh.flag, a.wait_ticks)) {
            // timed out: every segment still unpublished is computed -- with
            // the same lane mapping and arithmetic as its own workgroup -- and
            // published by the one workgroup that claims it; then all states
            // are collected.  Each segment is by then published or being
            // computed by a running workgroup that needs nothing from anyone,
            // so that wait ends; and however many workgroups time out, each
            // segment is read at most once more.
            __syncthreads();   // every lane has read collect's flag
            for (int s = 0; s < W; ++s) {
                if (threadIdx.x == 0) {
                    bool have = true;
                    for (int q = 0; q < kStateWords; ++q)
                        have = have && (__hip_atomic_load(rec64 + kStateWords * s + q, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT) >> 32) != 0;
                    uint32_t expected = 0u;
                    sh.flag = !have && __hip_atomic_compare_exchange_strong(rec + claim_word(W, s), &expected, 1u,
                                                                           __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                                           __HIP_MEMORY_SCOPE_AGENT);
                }
                __syncthreads();
                const bool mine = sh.flag != 0u;
                __syncthreads();
                if (mine) {
                    const int64_t o_u0 = s * kSegSpan;
                    const Stats ol = lane_state<BF16_IN, false, false, TOPK>(o_u0, units, c, tau, [&](int k, Unit<BF16_IN>& u) {
                        u.load(a, row_unit0 + lane_unit(o_u0, k), lane_unit(o_u0, k) < units);
                    });
                    publish(rec64, s, group_merge<kSegThreads>(ol, sh.part));
                }
            }
            collect(rec64, W, sh.seg_words, &sh.flag, ~(uint64_t)0);
        }
        row_st = merge_segments(sh.seg_words, W);
    }
    if (threadIdx.x == 0) sh.rk = row_const(row_st, c, a.inv_t, gmul, a.lgmul, GRAD != 0);
    __syncthreads();
    const RowConst k = sh.rk;
    if (k.form != FORM_LOSS) {
        if (seg == 0 && threadIdx.x == 0) a.row_loss[row] = k.loss;
        if constexpr (GRAD != 0) {
            if (k.form == FORM_PLAIN)
                seg_pass2<BF16_IN, GRAD, FULL, TOPK, FORM_PLAIN>(m, a, row_unit0, seg_u0, units, c, tau, k, kept_units);
            else
                seg_pass2<BF16_IN, GRAD, FULL, TOPK, FORM_SELECT>(m, a, row_unit0, seg_u0, units, c, tau, k, kept_units);
        }
        return;
    }
    const LossAcc acc = seg_pass2<BF16_IN, GRAD, FULL, TOPK, FORM_LOSS>(m, a, row_unit0, seg_u0, units, c, tau, k,
                                                                        kept_units);
    const LossSum part = group_sum<kSegThreads>(acc, sh.lpart);
    if (threadIdx.x == 0) {
        if (W == 1) {
            a.row_loss[row] = (float)termwise_kl(part.l, part.y, part.p);
        } else {
            double* share = reinterpret_cast<double*>(rec + share_word(W, seg));
            share[0] = part.l;
            share[1] = part.y;
            share[2] = part.p;
            if (seg == 0) {
                a.row_loss[row] = k.loss;
                rec[flag_word(W)] = 1u;
            }
        }
    }
}

__device__ __forceinline__ uint64_t* rec_of(uint32_t* rec_base, int64_t row, int W)
{
    return reinterpret_cast<uint64_t*>(rec_base + row * rec_words(W));
}

template <bool BF16_IN, int GRAD, bool FULL, bool TOPK>
__device__ __forceinline__ void seg_body(const KlArgs& a, int W, int64_t row, int seg, float c, float gmul,
                                         uint32_t* rec_base, SegShared& sh)
{
    const int64_t units = a.vocab >> 3;
    const int64_t seg_u0 = seg * kSegSpan;
    const float tau = TOPK ? a.tau[row] : 0.0f;
    SegRegs<BF16_IN> m;
    seg_load<BF16_IN, FULL>(m, a, row * units, seg_u0, units);
    uint32_t kept_units = 0u;   // TOPK: bit k set when the lane's unit k holds a kept entry
    const Stats st = seg_pass1<BF16_IN, FULL, TOPK>(m, seg_u0, units, c, tau, sh.part, &kept_units);
    if (W > 1) publish(rec_of(rec_base, row, W), seg, st);
    // From here on (the row's statistics, pass 2, the gradient stores) the
    // waves run at a raised priority: a workgroup that has its segment's
    // state out is served ahead of those still in pass 1, so it stores and
    // leaves sooner and its slot takes the next segment's loads (8192 x
    // 131072 bf16: 1.123 -> 1.105 ms; raising pass 1 instead, or the loads,
    // measured slower or no better).
    __builtin_amdgcn_s_setprio(2);
    seg_finish<BF16_IN, GRAD, FULL, TOPK>(m, a, W, row, seg, st, c, tau, gmul, rec_base, sh, kept_units);
}

// One workgroup per segment: load, pass 1, publish, wait, pass 2.  Segments
// that lie wholly inside the row (all but a ragged last one) take a form
// without per-unit bounds tests.
// TOPK: only the entries whose teacher logit is at least the row's threshold
// a.tau[row] count (the kept set of the teacher-top-k KL); gradient 0 elsewhere
template <bool BF16_IN, int GRAD, bool TOPK> // GRAD: 0 none, 1 bf16, 2 fp32
__device__ __forceinline__ void seg_entry(const KlArgs& a, int W, float c, float gmul, uint32_t* rec_base)
{
    __shared__ SegShared sh;
    const int64_t row = blockIdx.x / W;
    const int seg = (int)(blockIdx.x - row * W);
    if ((seg + 1) * kSegSpan <= (a.vocab >> 3))
        seg_body<BF16_IN, GRAD, true, TOPK>(a, W, row, seg, c, gmul, rec_base, sh);
    else
        seg_body<BF16_IN, GRAD, false, TOPK>(a, W, row, seg, c, gmul, rec_base, sh);
}

// bf16 logits: held to 128 VGPRs, four workgroups per CU
template <int GRAD, bool TOPK>
__global__ __launch_bounds__(kSegThreads, 4) void kl_seg_bf16_kernel(KlArgs a, int W, float c, float gmul,
                                                                     uint32_t* rec_base)
{
    seg_entry<true, GRAD, TOPK>(a, W, c, gmul, rec_base);
}

template <int GRAD, bool TOPK>
__global__ __launch_bounds__(kSegThreads) void kl_seg_f32_kernel(KlArgs a, int W, float c, float gmul,
                                                                 uint32_t* rec_base)
{
    seg_entry<false, GRAD, TOPK>(a, W, c, gmul, rec_base);
}

// ---------------------------------------------------------------------------
// Two-pass kernel for rows longer than kMaxSegments segments: one workgroup
// per row streams the row twice (online state, then the gradient and, on rows
// that take it, the term-wise KL).
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 1024;

// fold one unit of 8 teacher / student logits into the lane's running state
__device__ __forceinline__ void accumulate(Stats& st, const float (&t)[8], const float (&s)[8], float c)
{
    const float nmt = maxnan(st.mt, max8(t) * c);
    const float nms = maxnan(st.ms, max8(s) * c);
    const float ft = st.mt == nmt ? 1.0f : exp2_hw(st.mt - nmt);
    const float fs = st.ms == nms ? 1.0f : exp2_hw(st.ms - nms);
    st.mt = nmt;
    st.ms = nms;
    float et[8], es[8];
    float pa = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        et[i] = exp2_hw(__builtin_fmaf(t[i], c, -nmt));
        es[i] = exp2_hw(__builtin_fmaf(s[i], c, -nms));
        pa = __builtin_fmaf(et[i], t[i] - s[i], pa);
        st.dx = maxnan(st.dx, s[i] - t[i]);
    }
    st.zt = st.zt * ft + sum8(et);
    st.at = st.at * ft + pa;
    st.zs = st.zs * fs + sum8(es);
}

struct RowShared {
    Stats part[kRowThreads / 64];
    LossSum lpart[kRowThreads / 64];
    RowConst rk;
};

template <bool BF16_IN, int GRAD>
__global__ __launch_bounds__(kRowThreads) void kl_row_kernel(KlArgs a, float c, float gmul)
{
    __shared__ RowShared sh;
    const int64_t row = blockIdx.x;
    const int64_t units = a.vocab >> 3;
    const int64_t ubase = row * units;
    const int tid = threadIdx.x;
    Stats st = empty_stats();
    for (int64_t u = tid; u < units; u += kRowThreads) {
        float t[8], s[8];
        load8<BF16_IN>(a.teacher, ubase + u, true, t);
        load8<BF16_IN>(a.student, ubase + u, true, s);
        accumulate(st, t, s, c);
    }
    const Stats w = group_merge<kRowThreads>(st, sh.part);
    if (tid == 0) sh.rk = row_const(w, c, a.inv_t, gmul, a.lgmul, GRAD != 0);
    __syncthreads();
    const RowConst k = sh.rk;
    if (GRAD == 0 && k.form != FORM_LOSS) {
        if (tid == 0) a.row_loss[row] = k.loss;
        return;
    }
    LossAcc acc{0.0f, 0.0f, 0.0f};
    for (int64_t u = tid; u < units; u += kRowThreads) {
        float t[8], s[8];
        load8<BF16_IN>(a.teacher, ubase + u, true, t);
        load8<BF16_IN>(a.student, ubase + u, true, s);
        if (k.form == FORM_LOSS) unit_grad<GRAD, false, FORM_LOSS>(t, s, c, 0.0f, k, a, ubase + u, acc);
        else if (k.form == FORM_PLAIN) unit_grad<GRAD, false, FORM_PLAIN>(t, s, c, 0.0f, k, a, ubase + u, acc);
        else unit_grad<GRAD, false, FORM_SELECT>(t, s, c, 0.0f, k, a, ubase + u, acc);
    }
    if (k.form != FORM_LOSS) {
        if (tid == 0) a.row_loss[row] = k.loss;
        return;
    }
    const LossSum part = group_sum<kRowThreads>(acc, sh.lpart);
    if (tid == 0) a.row_loss[row] = (float)termwise_kl(part.l, part.y, part.p);
}

// Mean of the per-row losses, in two kernels and a fixed order.  Rows the
// segment kernels marked for the term-wise KL (rec non-null, W > 1) first
// get their loss from their segments' shares, added in segment order (also
// written to row_loss): one lane per row, kMeanRows rows per workgroup,
// whose binary64 sum (fixed tree) goes to partial[workgroup].  One
// workgroup then adds the partials: lane i takes partials i, i + 1024, ...
// in order, then a fixed tree.
constexpr int kMeanRows = 256;

__global__ __launch_bounds__(kMeanRows) void kl_row_finish_kernel(float* row_loss, int64_t rows, const uint32_t* rec,
                                                                  int W, double* partial)
{
    __shared__ double part[kMeanRows];
    const int64_t r = (int64_t)blockIdx.x * kMeanRows + threadIdx.x;
    double v = 0.0;
    if (r < rows) {
        float x = row_loss[r];
        if (rec) {
            const uint32_t* rr = rec + r * rec_words(W);
            if (rr[flag_word(W)]) {
                double l = 0.0, y = 0.0, p = 0.0;
                for (int seg = 0; seg < W; ++seg) {
                    const double* share = reinterpret_cast<const double*>(rr + share_word(W, seg));
                    l += share[0];
                    y += share[1];
                    p += share[2];
                }
                x = (float)termwise_kl(l, y, p);
                row_loss[r] = x;
            }
        }
        v = (double)x;
    }
    part[threadIdx.x] = v;
    __syncthreads();
    for (int w = kMeanRows / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[blockIdx.x] = part[0];
}

__global__ __launch_bounds__(1024) void kl_mean_kernel(const double* partial, int64_t groups, int64_t rows,
                                                       float* loss_out)
{
    __shared__ double part[1024];
    double acc = 0.0;
    for (int64_t i = threadIdx.x; i < groups; i += 1024) acc += partial[i];
    part[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) loss_out[0] = rows > 0 ? (float)(part[0] / (double)rows) : 0.0f;
}

// ---------------------------------------------------------------------------
// Teacher-top-k KL ([Qwen] "3. QAD": the distillation run restricts the KD
// loss to the teacher's top-4096 vocabulary entries; the page gives no tie
// rule and no normalisation).  Kept set of a row: every entry whose teacher
// logit is at least the k-th largest (ties kept); both softmaxes renormalised
// over it; gradient 0 elsewhere.  One workgroup of 1024 lanes per row:
//   1. the k-th largest teacher logit, exactly: radix select over
//      order-preserving integer keys (16-bit for bf16, 32-bit for fp32),
//      digits of up to 12 bits from the top; each round counts, in an LDS
//      histogram, the keys that match the digits chosen so far, and a suffix
//      scan over the bins picks the digit holding rank k;
//   2. the online softmax state of the kept entries, teacher and student;
//   3. the gradient (q~ - p~) grad_scale / T on kept entries, 0 elsewhere.
// Rows of at most kMaxSegments record segments split the work: a threshold
// kernel finds the k-th largest teacher logit per row (kl_sel16_kernel from
// exact key counts for bf16 teachers, kl_topk_tau_kernel by the radix rounds
// for fp32 ones and for bf16 rows whose counts overflow), then the one-pass
// segment kernels run masked by it (TOPK).  Longer rows take kl_topk_kernel,
// one workgroup per row that streams the row in every step.
// ---------------------------------------------------------------------------
constexpr int kTopThreads = 1024;
constexpr int kDigitBits = 12;

// order-preserving unsigned keys: a larger key is a larger value; -0 is
// folded onto +0 so that equal values have equal keys
__device__ __forceinline__ uint32_t key16(uint32_t h)
{
    h = h == 0x8000u ? 0u : h;
    return (h & 0x8000u) ? (h ^ 0xFFFFu) : (h | 0x8000u);
}

__device__ __forceinline__ uint32_t key32(uint32_t u)
{
    u = u == 0x80000000u ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <bool BF16>
__device__ __forceinline__ void teacher_keys(const Unit<BF16>& u, uint32_t (&k)[8])
{
    if constexpr (BF16) {
        const uint32_t w[4] = {u.t[0].x, u.t[0].y, u.t[0].z, u.t[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { k[2 * i] = key16(w[i] & 0xFFFFu); k[2 * i + 1] = key16(w[i] >> 16); }
    } else {
        const uint32_t w[8] = {u.t[0].x, u.t[0].y, u.t[0].z, u.t[0].w, u.t[1].x, u.t[1].y, u.t[1].z, u.t[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) k[i] = key32(w[i]);
    }
}

struct TopShared {
    uint32_t hist[1 << kDigitBits];
    uint32_t wave_tot[kTopThreads / 64];
    uint32_t digit, above;
    Stats part[kTopThreads / 64];
    LossSum lpart[kTopThreads / 64];
    RowConst rk;
};

// inclusive prefix sum over the workgroup's lanes in lane order
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wave_tot)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t n = __shfl_up(v, o, 64);
        if (lane >= o) v += n;
    }
    if (lane == 63) wave_tot[w] = v;
    __syncthreads();
    uint32_t off = 0;
    for (int i = 0; i < w; ++i) off += wave_tot[i];
    __syncthreads();
    return v + off;
}

// the key of the k-th largest teacher logit of the row (1 <= k <= vocab);
// for_t(f) calls f(unit, valid) for each of the lane's teacher units
template <bool BF16, class ForT>
__device__ uint32_t kth_largest_key(uint32_t k, ForT for_t, TopShared& sh)
{
    constexpr int KB = BF16 ? 16 : 32;
    uint32_t prefix = 0, remaining = k;
    for (int used = 0; used < KB;) {
        const int d = KB - used < kDigitBits ? KB - used : kDigitBits;
        const int nb = 1 << d, shift = KB - used - d;
        for (int i = threadIdx.x; i < nb; i += kTopThreads) sh.hist[i] = 0u;
        __syncthreads();
        for_t([&](const Unit<BF16>& u, bool valid) {
            if (!valid) return;
            uint32_t key[8];
            teacher_keys<BF16>(u, key);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (used == 0 || (key[i] >> (KB - used)) == prefix) atomicAdd(&sh.hist[(key[i] >> shift) & (nb - 1)], 1u);
        });
        __syncthreads();
        // lane l sums the g bins below nb - l g (from the top), then a scan
        // gives every group the count above it; one group holds rank k
        const int g = nb >= kTopThreads ? nb / kTopThreads : 1;
        const int groups = nb / g;
        const int top = nb - 1 - (int)threadIdx.x * g;
        uint32_t local = 0;
        if ((int)threadIdx.x < groups)
            for (int b = 0; b < g; ++b) local += sh.hist[top - b];
        const uint32_t incl = block_incl_scan(local, sh.wave_tot);
        if ((int)threadIdx.x < groups && incl - local < remaining && remaining <= incl) {
            uint32_t cum = incl - local;
            for (int b = 0; b < g; ++b) {
                const uint32_t h = sh.hist[top - b];
                if (remaining <= cum + h) {
                    sh.digit = (uint32_t)(top - b);
                    sh.above = cum;
                    break;
                }
                cum += h;
            }
        }
        __syncthreads();
        prefix = (prefix << d) | sh.digit;
        remaining -= sh.above;
        used += d;
        __syncthreads();  // hist, digit and above are rewritten next round
    }
    return prefix;
}

// the key of a logit value (the value is a bf16 value when BF16)
template <bool BF16>
__device__ __forceinline__ uint32_t key_of_value(float v)
{
    return BF16 ? key16(as_u(v) >> 16) : key32(as_u(v));
}

// the value whose key is `key` (inverse of key16 / key32)
template <bool BF16>
__device__ __forceinline__ float value_of_key(uint32_t key)
{
    if constexpr (BF16) {
        const uint32_t h = (key & 0x8000u) ? (key ^ 0x8000u) : (key ^ 0xFFFFu);
        return as_f(h << 16);
    } else {
        return as_f((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
    }
}

template <bool BF16_IN, int GRAD>
__global__ __launch_bounds__(kTopThreads) void kl_topk_kernel(KlArgs a, uint32_t k, float c, float gmul)
{
    __shared__ TopShared sh;
    const int64_t row = blockIdx.x;
    const int64_t units = a.vocab >> 3;
    const int64_t ubase = row * units;
    const int UL = (int)((units + kTopThreads - 1) / kTopThreads);
    const int tid = threadIdx.x;

    // f(teacher unit, valid) over the lane's units
    auto for_t = [&](auto f) {
#pragma unroll 4
        for (int j = 0; j < UL; ++j) {
            const int64_t u = (int64_t)j * kTopThreads + tid;
            Unit<BF16_IN> un;
            un.load(a, ubase + u, u < units);
            f(un, u < units);
        }
    };
    // the threshold key: given (a.tau, as a logit value) or selected here
    const uint32_t tau = a.tau ? key_of_value<BF16_IN>(a.tau[row]) : kth_largest_key<BF16_IN>(k, for_t, sh);

    // f(teacher and student unit, valid, unit index) over the lane's units
    auto for_ts = [&](auto f) {
#pragma unroll 4
        for (int j = 0; j < UL; ++j) {
            const int64_t u = (int64_t)j * kTopThreads + tid;
            Unit<BF16_IN> un;
            un.load(a, ubase + u, u < units);
            f(un, u < units, ubase + u);
        }
    };

    // kept-set softmax state, online as in the full-vocabulary kernel
    float mt = -__builtin_inff(), ms = -__builtin_inff(), zt = 0.0f, zs = 0.0f, at = 0.0f, dx = -__builtin_inff();
    for_ts([&](const Unit<BF16_IN>& both, bool valid, int64_t) {
        if (!valid) return;
        uint32_t key[8];
        teacher_keys<BF16_IN>(both, key);
        float tv[8], sv[8], pt[8], ps[8];
        both.values(tv, sv);
        float umt = -__builtin_inff(), ums = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (key[i] >= tau) { umt = maxnan(umt, tv[i]); ums = maxnan(ums, sv[i]); }
        }
        const float nmt = maxnan(mt, umt * c), nms = maxnan(ms, ums * c);
        const float ft = nmt == mt ? 1.0f : exp2_hw(mt - nmt);
        const float fs = nms == ms ? 1.0f : exp2_hw(ms - nms);
        mt = nmt;
        ms = nms;
        float pa = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool kept = key[i] >= tau;
            pt[i] = kept ? exp2_hw(__builtin_fmaf(tv[i], c, -mt)) : 0.0f;
            ps[i] = kept ? exp2_hw(__builtin_fmaf(sv[i], c, -ms)) : 0.0f;
            pa = kept ? __builtin_fmaf(pt[i], tv[i] - sv[i], pa) : pa;
            dx = kept ? maxnan(dx, sv[i] - tv[i]) : dx;
        }
        zt = zt * ft + sum8(pt);
        at = at * ft + pa;
        zs = zs * fs + sum8(ps);
    });
    const Stats row_st = group_merge<kTopThreads>(Stats{mt, zt, at, ms, zs, dx}, sh.part);
    if (tid == 0) sh.rk = row_const(row_st, c, a.inv_t, gmul, a.lgmul, GRAD != 0);
    __syncthreads();
    const RowConst rk = sh.rk;
    if (GRAD == 0 && rk.form != FORM_LOSS) {
        if (tid == 0) a.row_loss[row] = rk.loss;
        return;
    }
    // the kept set as a value test (keys fold -0 onto +0, as the comparison does)
    const float tau_v = value_of_key<BF16_IN>(tau);
    LossAcc acc{0.0f, 0.0f, 0.0f};
    for_ts([&](const Unit<BF16_IN>& both, bool valid, int64_t u) {
        if (!valid) return;
        float tv[8], sv[8];
        both.values(tv, sv);
        if (rk.form == FORM_LOSS) unit_grad<GRAD, true, FORM_LOSS>(tv, sv, c, tau_v, rk, a, u, acc);
        else if (rk.form == FORM_PLAIN) unit_grad<GRAD, true, FORM_PLAIN>(tv, sv, c, tau_v, rk, a, u, acc);
        else unit_grad<GRAD, true, FORM_SELECT>(tv, sv, c, tau_v, rk, a, u, acc);
    });
    if (rk.form != FORM_LOSS) {
        if (tid == 0) a.row_loss[row] = rk.loss;
        return;
    }
    const LossSum part = group_sum<kTopThreads>(acc, sh.lpart);
    if (tid == 0) a.row_loss[row] = (float)termwise_kl(part.l, part.y, part.p);
}


// Threshold of the teacher-top-k KL for the segment kernels: tau_out[row] =
// the k-th largest teacher logit of the row (the radix select above), the
// teacher row streamed once per round.  (Holding a 128K-logit row in
// registers allows one 1024-lane workgroup per CU and measured slower than
// two streaming ones, whose loads and LDS histograms overlap.)  REDO: only
// the rows kl_sel16_kernel left NaN (their key counts overflowed).
template <bool BF16, bool REDO = false>
__global__ __launch_bounds__(kTopThreads) void kl_topk_tau_kernel(const void* teacher, int64_t vocab, uint32_t k,
                                                                  float* tau_out)
{
    __shared__ TopShared sh;
    if (REDO && !__builtin_isnan(tau_out[blockIdx.x])) return;   // only rows the count kernel left NaN
    constexpr int V = Unit<BF16>::V;
    const int64_t row = blockIdx.x;
    const int64_t units = vocab >> 3;
    const int64_t ubase = row * units;
    const int UL = (int)((units + kTopThreads - 1) / kTopThreads);
    const int tid = threadIdx.x;
    auto for_t = [&](auto f) {
#pragma unroll 4
        for (int j = 0; j < UL; ++j) {
            const int64_t u = (int64_t)j * kTopThreads + tid;
            Unit<BF16> un;
#pragma unroll
            for (int q = 0; q < V; ++q) un.t[q] = u < units ? ldnt(teacher, V * (ubase + u) + q) : v4u{0u, 0u, 0u, 0u};
            f(un, u < units);
        }
    };
    const uint32_t key = kth_largest_key<BF16>(k, for_t, sh);
    if (tid == 0) tau_out[row] = value_of_key<BF16>(key);
}

// ---------------------------------------------------------------------------
// Teacher-top-p (nucleus) threshold ([Qwen] "3. QAD" names top-p as the
// variant to try after the top-k run).  tau_out[row] = the largest teacher
// value at which the teacher mass of the entries at or above it reaches
// top_p; top_p >= 1 keeps every entry (tau = the smallest value).  Masses are
// p_v up to the row's common factor: w_v = 2^(c t_v - m), m = RN(c max t),
// exactly the exponentials of the KL kernels, taken in fixed point
// (floor(w 2^40) in 64-bit integers) so that every sum is exact and
// independent of the order of the LDS atomics:
//   0. the row's largest key (integer max), hence m;
//   1. a radix round over the top 12 key bits: an LDS histogram sums the
//      fixed-point masses per digit; its total is Z, the target is
//      ceil(top_p Z), and a scan from the top finds the digit at which the
//      accumulated mass reaches it;
//   2. further rounds resolve the remaining key bits inside that digit.
// Weights below 2^-40 of the largest count as 0 (at most vocab * 2^-40 of the
// mass).  The teacher row is streamed once per step: three times for bf16,
// four for fp32.
// ---------------------------------------------------------------------------
// floor(w 2^40) as a 64-bit integer, w in [0, 2]: w 2^40 is an exact float
// with at most 24 significant bits, split exactly into its high and low
// 32-bit parts (the same value as a plain truncating conversion)
__device__ __forceinline__ unsigned long long fix40(float w)
{
    const float x = w * 0x1p40f;
    const uint32_t hi = (uint32_t)(x * 0x1p-32f);
    const uint32_t lo = (uint32_t)__builtin_fmaf((float)hi, -0x1p32f, x);
    return ((unsigned long long)hi << 32) | lo;
}

struct TopPShared {
    unsigned long long hist[1 << kDigitBits];
    unsigned long long wave_tot[kTopThreads / 64];
    unsigned long long above, target;
    uint32_t digit;
    uint32_t wave_key[kTopThreads / 64];
};

__device__ __forceinline__ unsigned long long block_incl_scan64(unsigned long long v, unsigned long long* wave_tot)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long n = __shfl_up(v, o, 64);
        if (lane >= o) v += n;
    }
    if (lane == 63) wave_tot[w] = v;
    __syncthreads();
    unsigned long long off = 0;
    for (int i = 0; i < w; ++i) off += wave_tot[i];
    __syncthreads();
    return v + off;
}

template <bool BF16>
__device__ __forceinline__ void teacher_values(const Unit<BF16>& u, float (&tv)[8])
{
    if constexpr (BF16) {
        unpack8(u.t[0], tv);
    } else {
        tv[0] = as_f(u.t[0].x); tv[1] = as_f(u.t[0].y); tv[2] = as_f(u.t[0].z); tv[3] = as_f(u.t[0].w);
        tv[4] = as_f(u.t[1].x); tv[5] = as_f(u.t[1].y); tv[6] = as_f(u.t[1].z); tv[7] = as_f(u.t[1].w);
    }
}

// largest (MAX) or smallest key of the row, in every lane
template <bool BF16, bool MAX, class ForT>
__device__ uint32_t extreme_key(ForT for_t, uint32_t* wave_key)
{
    uint32_t e = MAX ? 0u : 0xFFFFFFFFu;
    for_t([&](const Unit<BF16>& u, bool valid) {
        if (!valid) return;
        uint32_t key[8];
        teacher_keys<BF16>(u, key);
#pragma unroll
        for (int i = 0; i < 8; ++i) e = MAX ? umax(e, key[i]) : min(e, key[i]);
    });
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t n = __shfl_xor(e, o, 64);
        e = MAX ? umax(e, n) : min(e, n);
    }
    if ((threadIdx.x & 63) == 0) wave_key[threadIdx.x >> 6] = e;
    __syncthreads();
    e = wave_key[0];
    for (int i = 1; i < kTopThreads / 64; ++i) e = MAX ? umax(e, wave_key[i]) : min(e, wave_key[i]);
    __syncthreads();
    return e;
}

// the key of the nucleus threshold (0 < top_p < 1); m = RN(c max t)
template <bool BF16, class ForT>
__device__ uint32_t nucleus_key(float top_p, float c, float m, ForT for_t, TopPShared& sh)
{
    constexpr int KB = BF16 ? 16 : 32;
    uint32_t prefix = 0;
    unsigned long long remaining = 0;
    for (int used = 0; used < KB;) {
        const int d = KB - used < kDigitBits ? KB - used : kDigitBits;
        const int nb = 1 << d, shift = KB - used - d;
        for (int i = threadIdx.x; i < nb; i += kTopThreads) sh.hist[i] = 0ull;
        __syncthreads();
        for_t([&](const Unit<BF16>& u, bool valid) {
            if (!valid) return;
            uint32_t key[8];
            float tv[8];
            teacher_keys<BF16>(u, key);
            teacher_values<BF16>(u, tv);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (used == 0 || (key[i] >> (KB - used)) == prefix) {
                    const unsigned long long w = fix40(exp2_hw(__builtin_fmaf(tv[i], c, -m)));
                    if (w) atomicAdd(&sh.hist[(key[i] >> shift) & (nb - 1)], w);
                }
            }
        });
        __syncthreads();
        // lane l sums the g bins below nb - l g (from the top), then a scan
        // gives every group the mass above it
        const int g = nb >= kTopThreads ? nb / kTopThreads : 1;
        const int groups = nb / g;
        const int top = nb - 1 - (int)threadIdx.x * g;
        unsigned long long local = 0;
        if ((int)threadIdx.x < groups)
            for (int b = 0; b < g; ++b) local += sh.hist[top - b];
        const unsigned long long incl = block_incl_scan64(local, sh.wave_tot);
        if (used == 0) {
            // the last lane's inclusive sum is the row's total mass Z
            if (threadIdx.x == kTopThreads - 1) {
                unsigned long long t = (unsigned long long)ceil((double)top_p * (double)incl);
                t = t > incl ? incl : t;
                sh.target = t < 1ull ? 1ull : t;
            }
            __syncthreads();
            remaining = sh.target;
        }
        if ((int)threadIdx.x < groups && incl - local < remaining && remaining <= incl) {
            unsigned long long cum = incl - local;
            for (int b = 0; b < g; ++b) {
                const unsigned long long h = sh.hist[top - b];
                if (remaining <= cum + h) {
                    sh.digit = (uint32_t)(top - b);
                    sh.above = cum;
                    break;
                }
                cum += h;
            }
        }
        __syncthreads();
        prefix = (prefix << d) | sh.digit;
        remaining -= sh.above;
        used += d;
        __syncthreads();  // hist, digit and above are rewritten next round
    }
    return prefix;
}

// REDO: only the rows kl_sel16_kernel left NaN (their key counts overflowed)
template <bool BF16, bool REDO = false>
__global__ __launch_bounds__(kTopThreads) void kl_topp_tau_kernel(const void* teacher, int64_t vocab, float top_p,
                                                                  float c, float* tau_out)
{
    __shared__ TopPShared sh;
    if (REDO && !__builtin_isnan(tau_out[blockIdx.x])) return;   // only rows the count kernel left NaN
    constexpr int V = Unit<BF16>::V;
    const int64_t row = blockIdx.x;
    const int64_t units = vocab >> 3;
    const int64_t ubase = row * units;
    const int UL = (int)((units + kTopThreads - 1) / kTopThreads);
    const int tid = threadIdx.x;
    auto for_t = [&](auto f) {
#pragma unroll 4
        for (int j = 0; j < UL; ++j) {
            const int64_t u = (int64_t)j * kTopThreads + tid;
            Unit<BF16> un;
#pragma unroll
            for (int q = 0; q < V; ++q) un.t[q] = u < units ? ldnt(teacher, V * (ubase + u) + q) : v4u{0u, 0u, 0u, 0u};
            f(un, u < units);
        }
    };
    uint32_t key;
    if (top_p >= 1.0f) {
        key = extreme_key<BF16, false>(for_t, sh.wave_key);
    } else {
        const float m = value_of_key<BF16>(extreme_key<BF16, true>(for_t, sh.wave_key)) * c;
        key = nucleus_key<BF16>(top_p, c, m, for_t, sh);
    }
    if (tid == 0) tau_out[row] = value_of_key<BF16>(key);
}

// ---------------------------------------------------------------------------
// Thresholds of bf16 rows in one read of the teacher.  A bf16 logit is one of
// 65536 keys and equal keys are equal values, so the count of every key
// determines the k-th largest value exactly, and, since the entries of one
// key share one fixed-point weight floor(2^(c v - m) 2^40), the nucleus too
// (the same integer sums as the radix rounds above, so the same choice).  The
// counts live in LDS as 16-bit halves of 32768 words (128 KiB; ds_add without
// return).  A half that passes 65535 carries into its neighbour or out of
// the word, which can only lower the sum of all halves, so a sum different
// from the row length (more than 65535 equal logits in the row) leaves the
// row's threshold NaN, and the radix kernel launched next redoes exactly
// those rows.  The per-row scan of the counts is spread over the whole
// workgroup (a row's distinct values crowd into the keys of a few lanes).
// ---------------------------------------------------------------------------
constexpr int kSelWords = 32768;        // two 16-bit counters per word
constexpr int kSelKeysPerLane = 65536 / kTopThreads;

struct alignas(16) SelShared {
    struct {
        uint32_t hist[kSelWords];
        unsigned long long mass[kTopThreads];   // top-p: the teacher mass of each lane's keys
        unsigned long long wave_tot64[kTopThreads / 64];
        uint32_t wave_tot[kTopThreads / 64];
        uint32_t wave_key[kTopThreads / 64];
        uint32_t wave_grp[kTopThreads / 64];      // top-p: which 32-lane groups hold counts
        unsigned long long total64, target, rem64;
        uint32_t total, key, lane, rem;
    } c;
};

// This kernel's keys: 0x8000 plus the bf16's sign-magnitude bits read as a
// two's-complement integer (order-preserving; -0 and +0 both give 0x8000;
// finite values give 1 .. 0xFFFF), a few integer operations without compares.
// Only threshold values leave the kernel, so its keys need not match the
// radix kernels' ones.
__device__ __forceinline__ uint32_t sel_key_lo(uint32_t w)   // the bf16 in bits 0..15
{
    const int32_t mag = (int32_t)(w & 0x7FFFu), s = (int32_t)(w << 16) >> 31;
    return (uint32_t)(((mag ^ s) - s) + 0x8000);
}
__device__ __forceinline__ uint32_t sel_key_hi(uint32_t w)   // the bf16 in bits 16..31
{
    const int32_t mag = (int32_t)((w >> 16) & 0x7FFFu), s = (int32_t)w >> 31;
    return (uint32_t)(((mag ^ s) - s) + 0x8000);
}
__device__ __forceinline__ float sel_value(uint32_t key)
{
    const int32_t v = (int32_t)key - 0x8000;
    const uint32_t h = v >= 0 ? (uint32_t)v : (0x8000u | (uint32_t)(-v));
    return as_f(h << 16);
}

__device__ __forceinline__ uint32_t sel_count(const uint32_t* hist, uint32_t key)
{
    return (hist[key >> 1] >> ((key & 1u) * 16u)) & 0xFFFFu;
}

// count the 8 teacher keys of one unit (16 bytes of bf16) into the histogram
__device__ __forceinline__ void sel_count_unit(uint32_t* hist, const v4u& v)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t k0 = sel_key_lo(w[i]), k1 = sel_key_hi(w[i]);
        atomicAdd(&hist[k0 >> 1], 1u + (k0 & 1u) * 0xFFFFu);   // 1 or 1 << 16
        atomicAdd(&hist[k1 >> 1], 1u + (k1 & 1u) * 0xFFFFu);
    }
}

// The threshold key of a row from its counted histogram (TOPP: the nucleus of
// mass top_p, top_p >= 1 the smallest key; else the k-th largest), or
// 0xFFFFFFFF when a counter overflowed.
template <bool TOPP>
__device__ uint32_t sel16_key(int64_t vocab, uint32_t k, float top_p, float c, SelShared& sh)
{
    const int tid = threadIdx.x;
    // lane l owns the kSelKeysPerLane keys below 65536 - kSelKeysPerLane l:
    // 32 words, contiguous and 128-byte aligned, read as eight 16-byte
    // vectors starting at a lane-dependent one so that the lanes of a wave
    // spread over the LDS banks
    constexpr int kWordsPerLane = kSelKeysPerLane / 2;
    static_assert(kWordsPerLane == 32, "eight 16-byte reads per lane");
    const uint32_t hi = 65535u - (uint32_t)tid * kSelKeysPerLane;
    const uint32_t whi = hi >> 1;
    const v4u* lane_words = reinterpret_cast<const v4u*>(sh.c.hist) + (whi - 31u) / 4u;
    uint32_t local = 0, nz = 0;   // nz bit o: word whi - o holds a count
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t cc = (uint32_t)(c + tid) & 7u;
        const v4u v = lane_words[cc];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            local += (w[i] & 0xFFFFu) + (w[i] >> 16);
            nz |= (w[i] != 0u ? 1u : 0u) << (31u - (4u * cc + (uint32_t)i));
        }
    }
    const uint32_t incl = block_incl_scan(local, sh.c.wave_tot);
    if (tid == kTopThreads - 1) sh.c.total = incl;
    __syncthreads();
    if ((int64_t)sh.c.total != vocab) return 0xFFFFFFFFu;   // a counter overflowed
    if constexpr (!TOPP) {
        // the lane whose keys hold rank k, then its 64 keys across wave 0
        if (incl - local < k && k <= incl) { sh.c.lane = (uint32_t)tid; sh.c.rem = k - (incl - local); }
        __syncthreads();
        if (tid < 64) {
            const uint32_t key = 65535u - sh.c.lane * kSelKeysPerLane - (uint32_t)tid;
            uint32_t v = sel_count(sh.c.hist, key);
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t n = __shfl_up(v, o, 64);
                if (tid >= o) v += n;
            }
            const unsigned long long hit = __ballot(v >= sh.c.rem);
            if (tid == 0) sh.c.key = 65535u - sh.c.lane * kSelKeysPerLane - (uint32_t)__builtin_ctzll(hit);
        }
        __syncthreads();
        return sh.c.key;
    } else {
        // the largest (smallest for top_p >= 1) key present.  Bit o of nz is
        // word whi - o, so the lane's highest (lowest) counted word is one
        // count of zeros away, and one read of it picks the key inside.
        const bool want_min = top_p >= 1.0f;
        uint32_t e = want_min ? 0xFFFFFFFFu : 0u;
        if (nz) {
            const uint32_t o = want_min ? 31u - (uint32_t)__builtin_clz(nz) : (uint32_t)__builtin_ctz(nz);
            const uint32_t wi = whi - o, w = sh.c.hist[wi];
            e = want_min ? ((w & 0xFFFFu) ? 2u * wi : 2u * wi + 1u) : ((w >> 16) ? 2u * wi + 1u : 2u * wi);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const uint32_t n = __shfl_xor(e, o, 64);
            e = want_min ? min(e, n) : umax(e, n);
        }
        // 32-lane groups (lanes 32 g .. 32 g + 31) whose words hold counts
        const unsigned long long act = __ballot(nz != 0u);
        if ((tid & 63) == 0) {
            const uint32_t wv = (uint32_t)tid >> 6;
            sh.c.wave_key[wv] = e;
            sh.c.wave_grp[wv] = ((uint32_t)act ? 1u : 0u) << (2 * wv) | ((uint32_t)(act >> 32) ? 1u : 0u) << (2 * wv + 1);
        }
        __syncthreads();
        e = sh.c.wave_key[0];
        uint32_t groups = sh.c.wave_grp[0];
        for (int i = 1; i < kTopThreads / 64; ++i) {
            e = want_min ? min(e, sh.c.wave_key[i]) : umax(e, sh.c.wave_key[i]);
            groups |= sh.c.wave_grp[i];
        }
        if (want_min) return e;
        const float m = sel_value(e) * c;
        // fixed-point mass of each key: count x floor(2^(c v - m) 2^40)
        auto key_mass = [&](uint32_t key, uint32_t n) {
            return fix40(exp2_hw(__builtin_fmaf(sel_value(key), c, -m))) * n;
        };
        // The mass of each lane's 32 words.  The distinct values of a row
        // crowd into a few thousand neighbouring keys, the words of a few
        // dozen lanes, so the work is spread instead: the 1024 words of group
        // g (lanes 32 g .. 32 g + 31 own them) are read one per lane, word
        // 1024 (31 - g) + t by lane t, and each 32-lane half of a wave, which
        // then holds the 32 words of one owner, sums them.  Only groups with
        // counts are visited (a handful per row); integer sums, so the totals
        // do not depend on the order.
        static_assert(kSelWords == kWordsPerLane * kTopThreads && kWordsPerLane == 32, "one group per round");
        for (uint32_t gm = groups; gm; gm &= gm - 1u) {
            const uint32_t j = 31u - (uint32_t)__builtin_ctz(gm);
            const uint32_t wi = j * (uint32_t)kTopThreads + (uint32_t)tid, w = sh.c.hist[wi];
            unsigned long long v = w ? key_mass(2u * wi, w & 0xFFFFu) + key_mass(2u * wi + 1u, w >> 16) : 0ull;
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
            if ((tid & 31) == 0) sh.c.mass[(uint32_t)(kTopThreads - 1) - (wi >> 5)] = v;
        }
        __syncthreads();
        const unsigned long long lm = (groups >> ((uint32_t)tid >> 5)) & 1u ? sh.c.mass[tid] : 0ull;
        const unsigned long long incl64 = block_incl_scan64(lm, sh.c.wave_tot64);
        if (tid == kTopThreads - 1) {
            unsigned long long t = (unsigned long long)ceil((double)top_p * (double)incl64);
            t = t > incl64 ? incl64 : t;
            sh.c.target = t < 1ull ? 1ull : t;
        }
        __syncthreads();
        const unsigned long long target = sh.c.target;
        if (incl64 - lm < target && target <= incl64) { sh.c.lane = (uint32_t)tid; sh.c.rem64 = target - (incl64 - lm); }
        __syncthreads();
        if (tid < 64) {
            const uint32_t key = 65535u - sh.c.lane * kSelKeysPerLane - (uint32_t)tid;
            unsigned long long v = key_mass(key, sel_count(sh.c.hist, key));
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const unsigned long long n = __shfl_up(v, o, 64);
                if (tid >= o) v += n;
            }
            const unsigned long long hit = __ballot(v >= sh.c.rem64);
            if (tid == 0) sh.c.key = 65535u - sh.c.lane * kSelKeysPerLane - (uint32_t)__builtin_ctzll(hit);
        }
        __syncthreads();
        return sh.c.key;
    }
}

// bf16 teacher rows: thresholds by the key counts (a row whose counters
// overflow is left NaN for the radix kernels).  One workgroup per CU (the histogram fills the LDS) walks rows
// r = blockIdx.x, + gridDim.x, ...; a lane streams its units in batches of
// kSelBatch with the next batch (the next row's first, across rows) in
// flight while it counts the current one and while the row is scanned.
constexpr int kSelBatch = 4;

template <bool TOPP>
__global__ __launch_bounds__(kTopThreads) void kl_sel16_kernel(const void* teacher, int64_t rows, int64_t vocab,
                                                               uint32_t k, float top_p, float c, float* tau_out)
{
    __shared__ SelShared sh;
    const int64_t units = vocab >> 3;
    const int tid = threadIdx.x;
    const int64_t per_batch = (int64_t)kSelBatch * kTopThreads;
    const int nbatch = (int)((units + per_batch - 1) / per_batch);
    auto load_batch = [&](int64_t row, int bi, v4u (&v)[kSelBatch]) {
#pragma unroll
        for (int q = 0; q < kSelBatch; ++q) {
            const int64_t u = (int64_t)bi * per_batch + (int64_t)q * kTopThreads + tid;
            v[q] = row < rows && u < units ? ldnt(teacher, row * units + u) : v4u{0u, 0u, 0u, 0u};
        }
    };
    v4u cur[kSelBatch], nxt[kSelBatch];
    int64_t row = blockIdx.x;
    load_batch(row, 0, cur);
    for (int i = tid; i < kSelWords / 4; i += kTopThreads) reinterpret_cast<v4u*>(sh.c.hist)[i] = v4u{0u, 0u, 0u, 0u};
    __syncthreads();
    for (; row < rows; row += gridDim.x) {
        for (int bi = 0; bi < nbatch; ++bi) {
            if (bi + 1 < nbatch) load_batch(row, bi + 1, nxt);
            else load_batch(row + gridDim.x, 0, nxt);
            // unrolled, the batch's units are read straight from registers
            // (a rolled loop indexes them dynamically, one move per word);
            // for top-p this adds spills in the per-row scan, which cost
            // less than the indexing in the counting loop did
#pragma unroll
            for (int q = 0; q < kSelBatch; ++q)
                if ((int64_t)bi * per_batch + (int64_t)q * kTopThreads + tid < units) sel_count_unit(sh.c.hist, cur[q]);
#pragma unroll
            for (int q = 0; q < kSelBatch; ++q) cur[q] = nxt[q];
        }
        __syncthreads();
        const uint32_t key = sel16_key<TOPP>(vocab, k, top_p, c, sh);
        // a counter overflowed (more than 65535 equal logits): NaN marks the
        // row for the streaming radix kernels launched after this one
        if (tid == 0) tau_out[row] = key == 0xFFFFFFFFu ? __builtin_nanf("") : sel_value(key);
        __syncthreads();
        for (int i = tid; i < kSelWords / 4; i += kTopThreads)
            reinterpret_cast<v4u*>(sh.c.hist)[i] = v4u{0u, 0u, 0u, 0u};
        __syncthreads();
    }
}

// clear every tag a launch waits on (the whole records)
__global__ void zero_records_kernel(uint32_t* rec, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
        rec[i] = 0u;
}

// the launch's scalars the row constants use: 1 / T and log2 |grad_scale / T|
KlArgs with_row_scales(const KlArgs& a)
{
    KlArgs b = a;
    b.inv_t = 1.0f / a.temperature;
    b.lgmul = (float)log2(fabs((double)a.grad_scale / (double)a.temperature));
    return b;
}

// segments of a row, kMaxSegments + 1 standing for "too many"
int segments(int64_t vocab)
{
    const int64_t w = ((vocab >> 3) + kSegSpan - 1) / kSegSpan;
    return (int)min(w, (int64_t)kMaxSegments + 1);
}

} // namespace

namespace {
inline size_t r256(size_t n) { return (n + 255) & ~(size_t)255; }
// workspace layout: per-row losses, per-row records, the mean's partial sums
size_t kl_recs_offset(int64_t tokens) { return r256((size_t)tokens * 4); }
size_t kl_partial_offset(int64_t tokens, int64_t vocab)
{
    const int W = segments(vocab);
    const size_t recs = W > 1 && W <= kMaxSegments ? (size_t)tokens * rec_words(W) * 4 : 0;
    return kl_recs_offset(tokens) + r256(recs);
}
} // namespace

size_t kl_workspace_bytes(int64_t tokens, int64_t vocab)
{
    const size_t groups = (size_t)((tokens + kMeanRows - 1) / kMeanRows);
    return kl_partial_offset(tokens, vocab) + r256(groups * 8);
}

namespace {

// the one-pass segment kernels (rows of at most kMaxSegments record segments)
// or the two-pass row kernel; TOPK: masked by a.tau
hipError_t launch_rows(const KlArgs& a0, void* workspace, bool topk, hipStream_t stream)
{
    const KlArgs a = with_row_scales(a0);
    const float c = kLog2e / a.temperature;
    const float gmul = a.grad_scale / a.temperature;
    const int W = segments(a.vocab);
    const int gmode = !a.grad ? 0 : a.grad_bf16 ? 1 : 2;
    uint32_t* rec = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + kl_recs_offset(a.tokens));
    if (W > 1 && W <= kMaxSegments) {
        const int64_t n = a.tokens * rec_words(W);
        hipLaunchKernelGGL(zero_records_kernel, dim3((unsigned)min((n + 255) / 256, (int64_t)65536)), dim3(256), 0,
                           stream, rec, n);
    }
    // rows in batches, so that no grid exceeds 2^22 workgroups
    const size_t in_row = (size_t)a.vocab * (a.bf16_in ? 2 : 4);
    const size_t g_row = (size_t)a.vocab * (a.grad_bf16 ? 2 : 4);
    const int64_t batch = W <= kMaxSegments ? ((int64_t)1 << 22) / W : (int64_t)1 << 20;
    for (int64_t r0 = 0; r0 < a.tokens; r0 += batch) {
        KlArgs b = a;
        b.tokens = min(batch, a.tokens - r0);
        b.teacher = static_cast<const char*>(a.teacher) + r0 * in_row;
        b.student = static_cast<const char*>(a.student) + r0 * in_row;
        b.row_loss = a.row_loss + r0;
        if (a.tau) b.tau = a.tau + r0;
        if (a.grad) b.grad = static_cast<char*>(a.grad) + r0 * g_row;
        if (W <= kMaxSegments) {
            uint32_t* brec = rec + r0 * rec_words(W);
            const dim3 grid((unsigned)(b.tokens * W)), block(kSegThreads);
#define KS(K, GM, TK) hipLaunchKernelGGL((K<GM, TK>), grid, block, 0, stream, b, W, c, gmul, brec)
#define KS3(K, TK) { if (gmode == 0) KS(K, 0, TK); else if (gmode == 1) KS(K, 1, TK); else KS(K, 2, TK); }
            if (a.bf16_in) { if (topk) KS3(kl_seg_bf16_kernel, true) else KS3(kl_seg_bf16_kernel, false) }
            else { if (topk) KS3(kl_seg_f32_kernel, true) else KS3(kl_seg_f32_kernel, false) }
#undef KS3
#undef KS
        } else {
            const dim3 grid((unsigned)b.tokens), block(kRowThreads);
#define KR(BF, GM) hipLaunchKernelGGL((kl_row_kernel<BF, GM>), grid, block, 0, stream, b, c, gmul)
            if (a.bf16_in) { if (gmode == 0) KR(true, 0); else if (gmode == 1) KR(true, 1); else KR(true, 2); }
            else { if (gmode == 0) KR(false, 0); else if (gmode == 1) KR(false, 1); else KR(false, 2); }
#undef KR
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// the mean kernel, after the row kernels; with the segment kernels' records
// (W > 1) it first completes the rows that took the term-wise KL
hipError_t launch_mean(const KlArgs& a, void* workspace, hipStream_t stream)
{
    const int W = a.tokens > 0 && a.vocab > 0 ? segments(a.vocab) : 0;
    char* ws = static_cast<char*>(workspace);
    const uint32_t* rec =
        W > 1 && W <= kMaxSegments ? reinterpret_cast<const uint32_t*>(ws + kl_recs_offset(a.tokens)) : nullptr;
    const int64_t groups = (a.tokens + kMeanRows - 1) / kMeanRows;
    double* partial = a.tokens > 0 ? reinterpret_cast<double*>(ws + kl_partial_offset(a.tokens, a.vocab)) : nullptr;
    if (groups > 0)
        hipLaunchKernelGGL(kl_row_finish_kernel, dim3((unsigned)groups), dim3(kMeanRows), 0, stream, a.row_loss,
                           a.tokens, rec, W, partial);
    hipLaunchKernelGGL(kl_mean_kernel, dim3(1), dim3(1024), 0, stream, partial, groups, a.tokens, a.loss_out);
    return hipGetLastError();
}

} // namespace

hipError_t launch_kl(const KlArgs& a, void* workspace, hipStream_t stream)
{
    if (a.tokens > 0 && a.vocab > 0) {
        KlArgs b = a;
        b.tau = nullptr;
        hipError_t e = launch_rows(b, workspace, false, stream);
        if (e != hipSuccess) return e;
    }
    return launch_mean(a, workspace, stream);
}

size_t kl_topk_workspace_bytes(int64_t tokens, int64_t vocab)
{
    return kl_workspace_bytes(tokens, vocab) + (((size_t)tokens * 4 + 255) & ~(size_t)255);
}

namespace {

// workgroups of the persistent bf16 threshold kernel: one per CU (cached per
// device), never more than rows
dim3 sel_grid(int64_t rows)
{
    static int cache[64];
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
        cus = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
        if (!cus && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
            __atomic_store_n(&cache[dev], cus, __ATOMIC_RELAXED);
    }
    if (cus <= 0) cus = 256;
    return dim3((unsigned)max((int64_t)1, min(rows, (int64_t)cus)));
}

// rows longer than kMaxSegments record segments: one workgroup per row
// streams it in every step (threshold from a.tau when given, else the k-th
// largest teacher logit)
hipError_t launch_topk_long_rows(const KlArgs& a0, uint32_t kk, hipStream_t stream)
{
    const KlArgs a = with_row_scales(a0);
    const float c = kLog2e / a.temperature;
    const float gmul = a.grad_scale / a.temperature;
    const int gmode = !a.grad ? 0 : a.grad_bf16 ? 1 : 2;
    const size_t in_row = (size_t)a.vocab * (a.bf16_in ? 2 : 4);
    const size_t g_row = (size_t)a.vocab * (a.grad_bf16 ? 2 : 4);
    const int64_t batch = (int64_t)1 << 20;
    for (int64_t r0 = 0; r0 < a.tokens; r0 += batch) {
        KlArgs b = a;
        b.tokens = min(batch, a.tokens - r0);
        b.teacher = static_cast<const char*>(a.teacher) + r0 * in_row;
        b.student = static_cast<const char*>(a.student) + r0 * in_row;
        b.row_loss = a.row_loss + r0;
        if (a.tau) b.tau = a.tau + r0;
        if (a.grad) b.grad = static_cast<char*>(a.grad) + r0 * g_row;
        const dim3 grid((unsigned)b.tokens), block(kTopThreads);
#define KT(BF, GM) hipLaunchKernelGGL((kl_topk_kernel<BF, GM>), grid, block, 0, stream, b, kk, c, gmul)
        if (a.bf16_in) { if (gmode == 0) KT(true, 0); else if (gmode == 1) KT(true, 1); else KT(true, 2); }
        else { if (gmode == 0) KT(false, 0); else if (gmode == 1) KT(false, 1); else KT(false, 2); }
#undef KT
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

} // namespace

hipError_t launch_kl_topk(const KlArgs& a, int64_t k, void* workspace, hipStream_t stream)
{
    if (a.tokens > 0 && a.vocab > 0) {
        const uint32_t kk = (uint32_t)(k < a.vocab ? k : a.vocab);
        KlArgs b = a;
        b.tau = nullptr;
        if (segments(a.vocab) <= kMaxSegments) {
            // thresholds, then the one-pass segment kernels masked by them
            float* tau = reinterpret_cast<float*>(static_cast<char*>(workspace) + kl_workspace_bytes(a.tokens, a.vocab));
            const int64_t batch = (int64_t)1 << 20;
            const size_t in_row = (size_t)a.vocab * (a.bf16_in ? 2 : 4);
            for (int64_t r0 = 0; r0 < a.tokens; r0 += batch) {
                const dim3 grid((unsigned)min(batch, a.tokens - r0)), block(kTopThreads);
                const void* t = static_cast<const char*>(a.teacher) + r0 * in_row;
                if (a.bf16_in) {
                    hipLaunchKernelGGL((kl_sel16_kernel<false>), sel_grid(min(batch, a.tokens - r0)), block, 0, stream, t,
                                       min(batch, a.tokens - r0), a.vocab, kk, 1.0f, 0.0f, tau + r0);
                    hipLaunchKernelGGL((kl_topk_tau_kernel<true, true>), grid, block, 0, stream, t, a.vocab, kk, tau + r0);
                } else hipLaunchKernelGGL((kl_topk_tau_kernel<false>), grid, block, 0, stream, t, a.vocab, kk, tau + r0);
                hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
            }
            b.tau = tau;
            hipError_t e = launch_rows(b, workspace, true, stream);
            if (e != hipSuccess) return e;
        } else {
            hipError_t e = launch_topk_long_rows(b, kk, stream);
            if (e != hipSuccess) return e;
        }
    }
    return launch_mean(a, workspace, stream);
}

hipError_t launch_kl_topp(const KlArgs& a, float top_p, float* tau_out, void* workspace, hipStream_t stream)
{
    if (a.tokens > 0 && a.vocab > 0) {
        // thresholds (into tau_out when given), then the masked KL
        float* tau = tau_out ? tau_out
                             : reinterpret_cast<float*>(static_cast<char*>(workspace) + kl_workspace_bytes(a.tokens, a.vocab));
        const float c = kLog2e / a.temperature;
        const int64_t batch = (int64_t)1 << 20;
        const size_t in_row = (size_t)a.vocab * (a.bf16_in ? 2 : 4);
        for (int64_t r0 = 0; r0 < a.tokens; r0 += batch) {
            const dim3 grid((unsigned)min(batch, a.tokens - r0)), block(kTopThreads);
            const void* t = static_cast<const char*>(a.teacher) + r0 * in_row;
            if (a.bf16_in) {
                hipLaunchKernelGGL((kl_sel16_kernel<true>), sel_grid(min(batch, a.tokens - r0)), block, 0, stream, t,
                                   min(batch, a.tokens - r0), a.vocab, 1u, top_p, c, tau + r0);
                hipLaunchKernelGGL((kl_topp_tau_kernel<true, true>), grid, block, 0, stream, t, a.vocab, top_p, c, tau + r0);
            } else hipLaunchKernelGGL((kl_topp_tau_kernel<false>), grid, block, 0, stream, t, a.vocab, top_p, c, tau + r0);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        KlArgs b = a;
        b.tau = tau;
        hipError_t e = segments(a.vocab) <= kMaxSegments ? launch_rows(b, workspace, true, stream)
                                                         : launch_topk_long_rows(b, 1u, stream);
        if (e != hipSuccess) return e;
    }
    return launch_mean(a, workspace, stream);
}

} // namespace qad
