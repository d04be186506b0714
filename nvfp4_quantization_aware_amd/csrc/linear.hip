// W4A4 NVFP4 fake-quant linear layer ([Qwen] "3. QAD": the student is the
// W4A4 NVFP4 model, weights and activations both NVFP4; [Lightning]
// "QAD的工作原理": simulated quantization runs in every student forward).
//
//   forward : y = QDQ(x) QDQ(w)^T        x [M][K], w [N][K], y [M][N]
//   backward: grad_x = grad_y QDQ(w),    grad_w = grad_y^T QDQ(x)
//             (straight-through through both quantizers)
//
// The forward quantizes x and w once each with the library's quantizer
// (dynamic per-tensor scales, blocks of 16 along K, or frozen weight scales)
// into packed NVFP4 operands: E2M1 codes, E4M3 block scales and the tensor
// scale, 9/16 of a byte per element.  The three products are one hand-written
// MFMA GEMM: each workgroup owns a 256 x 256 (or 256 x 128) output tile and
// stages 64-deep slices of both operands into LDS, rebuilding the QDQ values
// bf16(dec(code) * s_eff) there exactly as the quantizer's own bf16 output is
// formed (FP4 decode, one binary32 product, nearest-even bf16); eight waves
// multiply them with v_mfma_f32_32x32x16_bf16 into fp32 accumulators.  So
// the operands cross HBM as 4-bit codes, never as bf16 QDQ copies.
#include "libqad.h"

#include <type_traits>

#include "qad_device.h"
#include "qad_internal.h"

namespace qad {
namespace {

constexpr int kBM = 256, kBK = 64;              // workgroup tile: 256 x BN (BN 256 or 128), 64-deep steps
constexpr int kThreads = 512;                    // eight waves, two per SIMD, 4 (M) x 2 (N) over the tile
constexpr int kWM = 4;                           // waves along M; each owns 256 / kWM rows of the tile
// LDS tile layouts, rows of 64 contraction values (bf16):
//   padded (SWZ false): row stride 72 (144 B); the fragment reads (lanes
//     0..31 on rows r0..r0+31 at one 16-byte chunk) and the row-major stores
//     are conflict-free;
//   swizzled (SWZ true, the kernels with a transposed operand): row stride
//     64 (128 B), chunk c of row r stored at c ^ (r % 8) ^ (r / 8 % 8).  The
//     fragment reads still see 8 consecutive rows on 8 distinct chunks, and
//     the transposed stores (16 lanes on rows 4 i + e, i = 0..15) land on
//     each chunk twice instead of 8 of them on one bank group (measured:
//     bank conflicts were half of grad_x's LDS time and two thirds of
//     grad_w's).  The forward keeps the padded layout, whose addresses cost
//     fewer registers in its 256-wide kernel.
template <bool SWZ> constexpr int lds_stride() { return SWZ ? kBK : kBK + 8; }

template <bool SWZ>
__device__ __forceinline__ int lds_pos(int row, int col)
{
    if constexpr (SWZ) {
        const int sw = (row & 7) ^ ((row >> 3) & 7);
        return row * kBK + ((((col >> 3) ^ sw) & 7) << 3) + (col & 7);
    } else {
        return row * (kBK + 8) + col;
    }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// How an operand of C[M][N] = sum_k A(m, k) B(n, k) is stored.  "K": rows of
// the operand's output index, the contraction contiguous ([rows][K]); "T":
// rows of the contraction index, the output contiguous ([K][rows]).  NVFP4
// operands are packed (codes, block scales of 16 consecutive elements along
// the storage row, tensor scale); bf16 ones are plain.
enum { OP_BF16_K = 0, OP_FP4_K = 1, OP_BF16_T = 2, OP_FP4_T = 3 };

struct Operand {
    const void* data;       // bf16 values, or NVFP4 codes (two per byte, even element low)
    const uint8_t* scales;  // NVFP4 E4M3 block scale codes
    const float* tscale;    // NVFP4 tensor scale
    int64_t ld;             // elements per storage row
    int64_t rows;           // extent of the output index (M for A, N for B)
};

struct GemmArgs {
    Operand a, b;
    uint16_t* c;            // bf16 [M][N]
    int64_t M, N, K;        // K: contraction length
    int tiles_m, tiles_n;
};

// A thread's share of one R x 64 tile of an operand (R output rows by 64
// contraction values, kThreads threads).
//   K forms: EPT consecutive contraction values of one output row: row
//            t / TPR, contraction [EPT (t % TPR), +EPT); BLK NVFP4 blocks
//   T forms: RPT contraction rows of 4 consecutive outputs: outputs
//            [4 (t % OG), +4), contraction [RPT (t / OG), +RPT)
template <int R> struct Share {
    static constexpr int EPT = R * kBK / kThreads, TPR = kBK / EPT, BLK = EPT / 16;
    static constexpr int OG = R / 4, RPT = kBK * OG / kThreads;
};

// Staging registers of that share.  Loaded values stay as loaded (no
// arithmetic on them before the decode), so a thread never waits on its
// prefetch before the step that decodes it.
template <int KIND, int R> struct Stage;
template <int R> struct Stage<OP_BF16_K, R> { u32x4 v[Share<R>::EPT / 8]; uint32_t ok; };
template <int R> struct Stage<OP_FP4_K, R> { u32x2 code[Share<R>::BLK]; uint32_t sc[Share<R>::BLK]; uint32_t ok; };
template <int R> struct Stage<OP_BF16_T, R> { u32x2 v[Share<R>::RPT]; uint32_t ok; };
template <int R> struct Stage<OP_FP4_T, R> { uint32_t code[Share<R>::RPT]; uint32_t sc[Share<R>::RPT]; uint32_t ok; };

__device__ __forceinline__ u32x4 ld16(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// Global loads of the tile whose output rows start at row0 and contraction at
// k0; what lies outside the operand reads as zeros (code 0 decodes to +0).
// FAST (chosen per launch): every row of every operand is aligned for the
// vector forms below -- NVFP4 rows hold whole 16-byte runs of codes (K % 32
// == 0), bf16 rows whole 16-byte (K form) or 8-byte (T form) runs -- so each
// load is one vector from a clamped address, with no branch around it (a
// branch there makes the compiler wait for every load in flight at the loop
// head); what lies outside the operand is zeroed when decoded.  Otherwise
// the element-by-element forms.  FULL (FAST too): every tile lies wholly
// inside both operands and K % 64 == 0, so nothing is clamped or masked (the
// masks are constants the compiler folds away).
template <int KIND, int R, bool FAST, bool FULL>
__device__ __forceinline__ void stage_load(Stage<KIND, R>& s, const Operand& op, int64_t row0, int64_t k0, int64_t K)
{
    static_assert(FAST || !FULL, "FULL implies FAST");
    using S = Share<R>;
    const int t = threadIdx.x;
    if constexpr (KIND == OP_BF16_K || KIND == OP_FP4_K) {
        const int64_t row = row0 + t / S::TPR;
        const int64_t kc = k0 + S::EPT * (t % S::TPR);
        const bool rv = FULL || row < op.rows;
        if constexpr (KIND == OP_BF16_K && FAST) {
            // K (the backward's N) % 8 == 0: a run of 8 lies wholly inside or
            // outside the row; bit q of ok marks the runs inside
            const int64_t rc = rv ? row : op.rows - 1;
            const uint16_t* p = static_cast<const uint16_t*>(op.data) + rc * op.ld;
            uint32_t ok = 0u;
#pragma unroll
            for (int q = 0; q < S::EPT / 8; ++q) {
                const int64_t k = kc + 8 * q;
                const bool in = FULL || (rv && k < K);
                s.v[q] = ld16(p + (in ? k : 0));
                ok |= (uint32_t)in << q;
            }
            s.ok = ok;
        } else if constexpr (KIND == OP_BF16_K) {
            // the contraction here is the backward's N, of any length: a run
            // of 8 is loaded as one vector only when 16-byte aligned and
            // wholly inside the row, else element by element up to its end
            const uint16_t* p = static_cast<const uint16_t*>(op.data) + row * op.ld + kc;
            const bool vec = (op.ld & 7) == 0;
            s.ok = ~0u;
#pragma unroll
            for (int q = 0; q < S::EPT / 8; ++q) {
                const int64_t k = kc + 8 * q;
                if (rv && vec && k + 8 <= K) {
                    s.v[q] = ld16(p + 8 * q);
                } else {
                    uint32_t w[4] = {0u, 0u, 0u, 0u};
                    if (rv)
                        for (int e = 0; e < 8; ++e)
                            if (k + e < K) w[e >> 1] |= (uint32_t)p[8 * q + e] << (16 * (e & 1));
                    s.v[q] = u32x4{w[0], w[1], w[2], w[3]};
                }
            }
        } else {
            // K % 16 == 0 here: whole blocks.  Every load is issued: a block
            // outside the operand reads from an address clamped into it (the
            // start of the row; the load may then run past the row or the
            // codes, but stays inside the packed buffer, whose scales and
            // tensor-scale line follow the codes), and bit b of `ok` tells
            // the decode to zero block b.  When rows hold a whole number of
            // the thread's runs (K % (16 BLK) == 0) the run's codes are 16-byte
            // loads and its BLK scale bytes one load into sc[0] (bit 8 of
            // ok); otherwise 8-byte code loads and single scale bytes.
            const int64_t rc = rv ? row : op.rows - 1;
            const int64_t kk = FULL || kc < K ? kc : 0;
            const uint8_t* codes = static_cast<const uint8_t*>(op.data) + rc * (op.ld >> 1) + (kk >> 1);
            const uint8_t* sc = op.scales + rc * (op.ld >> 4) + (kk >> 4);
            uint32_t ok = 0u;
#pragma unroll
            for (int b = 0; b < S::BLK; ++b) ok |= (uint32_t)(FULL || (rv && kc + 16 * b < K)) << b;
            if constexpr (S::BLK >= 2 && FAST) {
#pragma unroll
                for (int h = 0; h < S::BLK / 2; ++h) {
                    const u32x4 c = ld16(codes + 16 * h);
                    s.code[2 * h] = u32x2{c[0], c[1]};
                    s.code[2 * h + 1] = u32x2{c[2], c[3]};
                }
                if constexpr (S::BLK == 4)
                    s.sc[0] = *reinterpret_cast<const uint32_t*>(sc);
                else if constexpr (S::BLK == 2)
                    s.sc[0] = *reinterpret_cast<const uint16_t*>(sc);
#pragma unroll
                for (int b = 1; b < S::BLK; ++b) s.sc[b] = 0u;
                ok |= 0x100u;
            } else {
#pragma unroll
                for (int b = 0; b < S::BLK; ++b) {
                    s.code[b] = ld8(codes + 8 * b);
                    s.sc[b] = sc[b];
                }
            }
            s.ok = ok;
        }
    } else {
        const int64_t kr0 = k0 + S::RPT * (t / S::OG);
        const int64_t o = row0 + 4 * (t % S::OG);
        if constexpr (KIND == OP_BF16_T && FAST) {
            // the output extent (the backward's N) % 4 == 0: a run of 4 lies
            // wholly inside or outside; bit i of ok marks the rows inside
            const bool ov = FULL || o < op.rows;
            const int64_t oc = ov ? o : 0;
            uint32_t ok = 0u;
#pragma unroll
            for (int i = 0; i < S::RPT; ++i) {
                const int64_t kr = kr0 + i;
                const bool in = FULL || (ov && kr < K);
                s.v[i] = ld8(static_cast<const uint16_t*>(op.data) + (in ? kr : 0) * op.ld + oc);
                ok |= (uint32_t)in << i;
            }
            s.ok = ok;
        } else if constexpr (KIND == OP_BF16_T) {
            const bool vec = (op.ld & 3) == 0 && o + 4 <= op.rows;   // 8-byte aligned, wholly inside
            s.ok = ~0u;
#pragma unroll
            for (int i = 0; i < S::RPT; ++i) {
                const int64_t kr = kr0 + i;
                const uint16_t* p = static_cast<const uint16_t*>(op.data) + kr * op.ld + o;
                if (kr < K && vec) {
                    s.v[i] = ld8(p);
                } else {
                    uint32_t w[2] = {0u, 0u};
                    if (kr < K)
                        for (int e = 0; e < 4; ++e)
                            if (o + e < op.rows) w[e >> 1] |= (uint32_t)p[e] << (16 * (e & 1));
                    s.v[i] = u32x2{w[0], w[1]};
                }
            }
        } else {
            // four codes (2 bytes) and their block's scale per contraction
            // row; the output extent is a multiple of 16, so a run of 4 lies
            // wholly inside or outside (clamped addresses and a validity
            // mask, as for the K form)
            const bool ov = FULL || o < op.rows;
            const int64_t oc = ov ? o : op.rows - 4;
            uint32_t ok = 0u;
#pragma unroll
            for (int i = 0; i < S::RPT; ++i) {
                const int64_t kr = kr0 + i;
                const int64_t krc = FULL || kr < K ? kr : K - 1;
                s.code[i] = *reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(op.data) +
                                                               krc * (op.ld >> 1) + (oc >> 1));
                s.sc[i] = op.scales[krc * (op.ld >> 4) + (oc >> 4)];
                ok |= (uint32_t)(FULL || (ov && kr < K)) << i;
            }
            s.ok = ok;
        }
    }
}

// The QDQ value pair of two codes (as the quantizer forms y): exact decode,
// one binary32 product each with the block's effective scale, nearest-even bf16
template <int SEL>
__device__ __forceinline__ uint32_t qdq_pair(uint32_t codes, float s)
{
    float lo, hi;
    fp4_decode_pair<SEL>(codes, lo, hi);
    return pack_bf16x2(lo * s, hi * s);
}

__device__ __forceinline__ void lds_store16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Effective scale fl(dec(c) s_g) of block scale code c (0 <= c < 128), or 0
// for a block outside the operand (whose codes are then zeroed too).
// The E4M3 value by gfx950's FP8 conversion (exact on every non-NaN code,
// checked on every code against the format's definition), one instruction where
// the bit arithmetic took about eight; code 0x7F, outside the scale codes the
// library writes or accepts, keeps the integer decode's 480 so that the
// product always agrees with the quantizer's own dequantization.
__device__ __forceinline__ float block_scale(uint32_t c, float s_g, bool ok)
{
    const float dec = c == 0x7Fu ? 480.0f : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, false)[0];
    return ok ? dec * s_g : 0.0f;
}

// Decoded values of a transposed operand on their way into LDS: w[e][p] is
// output row 4 og + e, contraction rows 2 p and 2 p + 1 of the thread's run.
template <int R> struct TBuf { uint32_t w[4][Share<R>::RPT / 2]; };

// Registers -> LDS tile [R output rows][64 contraction] (bf16, laid out by lds_pos),
// in four parts (u = 0..3) so that the decode can be spread over the four
// 16-deep MFMA slices of a step.  A part of a K operand is a quarter of the
// thread's 8-value runs; one of a T operand decodes a quarter of its
// contraction-row pairs, and the last part stores the transposed rows.
template <int KIND, int R, bool SWZ>
__device__ __forceinline__ void stage_store_part(const Stage<KIND, R>& s, TBuf<R>& tb, uint16_t* lds, float s_g, int u)
{
    using S = Share<R>;
    const int t = threadIdx.x;
    if constexpr (KIND == OP_BF16_K || KIND == OP_FP4_K) {
        constexpr int RUNS = S::EPT / 8, UPP = (RUNS + 3) / 4;   // 8-value runs, per part
        const int drow = t / S::TPR, dcol = S::EPT * (t % S::TPR);
#pragma unroll
        for (int v = 0; v < UPP; ++v) {
            const int r = u * UPP + v;   // run index
            if (r >= RUNS) break;
            uint16_t* dst = lds + lds_pos<SWZ>(drow, dcol + 8 * r);
            if constexpr (KIND == OP_BF16_K) {
                const bool ok = (s.ok >> r) & 1u;
                const u32x4 v = s.v[r];
                lds_store16(dst, u32x4{ok ? v[0] : 0u, ok ? v[1] : 0u, ok ? v[2] : 0u, ok ? v[3] : 0u});
            } else {
                // block r / 2: its scale byte from the one scale load or its own
                const int b = r >> 1;
                const bool ok = (s.ok >> b) & 1u;
                const uint32_t sb = (s.ok & 0x100u) ? s.sc[0] >> (8 * b) : s.sc[b];
                const float se = block_scale(sb & 127u, s_g, ok);
                const uint32_t c = ok ? s.code[b][r & 1] : 0u;
                lds_store16(dst, u32x4{qdq_pair<0>(c, se), qdq_pair<1>(c, se), qdq_pair<2>(c, se), qdq_pair<3>(c, se)});
            }
        }
    } else {
        constexpr int PAIRS = S::RPT / 2, PPP = (PAIRS + 3) / 4;   // contraction-row pairs, per part
#pragma unroll
        for (int v = 0; v < PPP; ++v) {
            const int p = u * PPP + v;
            if (p >= PAIRS) break;
            if constexpr (KIND == OP_BF16_T) {
                const bool oka = (s.ok >> (2 * p)) & 1u, okb = (s.ok >> (2 * p + 1)) & 1u;
                const u32x2 a = oka ? s.v[2 * p] : u32x2{0u, 0u}, b = okb ? s.v[2 * p + 1] : u32x2{0u, 0u};
                tb.w[0][p] = (a[0] & 0xFFFFu) | (b[0] << 16);
                tb.w[1][p] = (a[0] >> 16) | (b[0] & 0xFFFF0000u);
                tb.w[2][p] = (a[1] & 0xFFFFu) | (b[1] << 16);
                tb.w[3][p] = (a[1] >> 16) | (b[1] & 0xFFFF0000u);
            } else {
                float x[2][4];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int i = 2 * p + r;
                    const bool ok = (s.ok >> i) & 1u;
                    const float se = block_scale(s.sc[i] & 127u, s_g, ok);
                    const uint32_t c = ok ? s.code[i] : 0u;
                    float lo, hi;
                    fp4_decode_pair<0>(c, lo, hi);
                    x[r][0] = lo * se;
                    x[r][1] = hi * se;
                    fp4_decode_pair<1>(c, lo, hi);
                    x[r][2] = lo * se;
                    x[r][3] = hi * se;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) tb.w[e][p] = pack_bf16x2(x[0][e], x[1][e]);
            }
        }
        if (u == 3) {
            // output row 4 og + e receives contraction [RPT cg, +RPT)
            const int row0 = 4 * (t % S::OG), col0 = S::RPT * (t / S::OG);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (S::RPT >= 8) {
#pragma unroll
                    for (int h = 0; h < S::RPT / 8; ++h)
                        lds_store16(lds + lds_pos<SWZ>(row0 + e, col0 + 8 * h),
                                    u32x4{tb.w[e][4 * h], tb.w[e][4 * h + 1], tb.w[e][4 * h + 2], tb.w[e][4 * h + 3]});
                } else {
                    // 8 bytes: half a chunk (col0 % 8 is 0 or 4)
                    *reinterpret_cast<u32x2*>(lds + lds_pos<SWZ>(row0 + e, col0)) = u32x2{tb.w[e][0], tb.w[e][1]};
                }
            }
        }
    }
}

template <int KIND, int R, bool SWZ>
__device__ __forceinline__ void stage_store(const Stage<KIND, R>& s, uint16_t* lds, float s_g)
{
    TBuf<R> tb;
#pragma unroll
    for (int u = 0; u < 4; ++u) stage_store_part<KIND, R, SWZ>(s, tb, lds, s_g, u);
}

// tile index of workgroup `bid`: consecutive workgroups go to different XCDs
// (eight of them), so each XCD is given a contiguous run of tiles, ordered in
// groups of GH tile rows so that a run shares operand tiles in its XCD's L2
template <int GH>
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn)
{
    const int total = tiles_m * tiles_n;
    int id = bid;
    if ((total & 7) == 0) id = (bid & 7) * (total >> 3) + (bid >> 3);
    const int per_group = GH * tiles_n;
    const int g = id / per_group, first = g * GH;
    const int gm = tiles_m - first < GH ? tiles_m - first : GH;
    const int r = id - g * per_group;
    tm = first + r % gm;
    tn = r / gm;
}

template <int KIND> __device__ __forceinline__ float tensor_scale(const Operand& op)
{
    return (KIND == OP_FP4_K || KIND == OP_FP4_T) ? *op.tscale : 0.0f;
}

// The fragments of one 16-deep slice ks for wave (wm, wn): A rows
// [TI 32 wm + 32 i, +32), B rows [BN/2 wn + 32 j, +32); lane l holds row
// l % 32, contraction [8 (l / 32), +8) of the slice (the MFMA operand layout)
constexpr int kTI = kBM / kWM / 32;   // MFMA tiles of a wave along M
template <int BN, bool SWZ>
__device__ __forceinline__ void load_frags(const uint16_t* la, const uint16_t* lb, int ks, bf16x8_t (&fa)[kTI],
                                           bf16x8_t (&fb)[BN / 64])
{
    const int l = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave % kWM, wn = wave / kWM;
    const int kcol = ks * 16 + 8 * (l >> 5);
#pragma unroll
    for (int i = 0; i < kTI; ++i)
        fa[i] = *reinterpret_cast<const bf16x8_t*>(la + lds_pos<SWZ>(wm * 32 * kTI + i * 32 + (l & 31), kcol));
#pragma unroll
    for (int j = 0; j < BN / 64; ++j)
        fb[j] = *reinterpret_cast<const bf16x8_t*>(lb + lds_pos<SWZ>(wn * (BN / 2) + j * 32 + (l & 31), kcol));
}

// An NVFP4 A operand stored [K][rows] is the weight of grad_x computed as
// grad_x^T = wq^T grad_y^T; that product's C is written transposed.
template <int KA> constexpr bool kTransposedOut = KA == OP_FP4_T;

// C[M][N] = sum_k A(m, k) B(n, k), bf16 out of fp32 accumulation in a fixed
// order (k ascending in steps of 64, each step's four 16-deep MFMAs in
// order).  One 256 x BN tile per workgroup of eight waves, two per SIMD;
// wave (wm, wn) owns rows [64 wm, +64) and columns [BN/2 wn, +BN/2) as
// 2 x BN/64 MFMA tiles of 32 x 32.  Two LDS buffers: while the waves
// multiply the tiles of step s from one buffer (the fragments of each
// 16-deep slice read while the previous slice's MFMAs run), each thread
// decodes its registers of step s + 1 into the other, one quarter per slice,
// and has the loads of step s + 2 in flight; one barrier per step separates
// the phases.  Past the last step the loads repeat the last slice and the
// decode fills the idle buffer, so the loop body has no branches.
template <int KA, int KB, int BN, bool FAST, bool FULL>
__global__ __launch_bounds__(kThreads) void w4a4_gemm_kernel(GemmArgs g)
{
    constexpr int TJ = BN / 64;
    constexpr bool SWZ = KA == OP_BF16_T || KA == OP_FP4_T || KB == OP_BF16_T || KB == OP_FP4_T;
    constexpr int kBufA = kBM * lds_stride<SWZ>(), kBufB = BN * lds_stride<SWZ>();
    __shared__ __align__(16) uint16_t lds[2 * (kBufA + kBufB)];

    // a bf16 A operand (grad_y^T for grad_w) moves 4x the bytes of an NVFP4
    // one per tile row: fewer tile rows in flight keep its rows in L2 (4
    // against 8 measured 10% faster for grad_y as A); with an NVFP4 A the
    // products are the same at 2 to 16 within 3%
    constexpr int GH = KA == OP_FP4_K || KA == OP_FP4_T ? 8 : 4;
    int tm, tn;
    tile_of<GH>(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * BN;
    const float sa = tensor_scale<KA>(g.a), sb = tensor_scale<KB>(g.b);
    const int l = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave % kWM, wn = wave / kWM;

    f32x16_t acc[kTI][TJ];
#pragma unroll
    for (int i = 0; i < kTI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16_t{};

    const int64_t steps = (g.K + kBK - 1) / kBK;
    const int64_t last = (steps - 1) * kBK;
    Stage<KA, kBM> ra[2];
    Stage<KB, BN> rb[2];
    stage_load<KA, kBM, FAST, FULL>(ra[0], g.a, m0, 0, g.K);
    stage_load<KB, BN, FAST, FULL>(rb[0], g.b, n0, 0, g.K);
    stage_load<KA, kBM, FAST, FULL>(ra[1], g.a, m0, kBK < last ? kBK : last, g.K);
    stage_load<KB, BN, FAST, FULL>(rb[1], g.b, n0, kBK < last ? kBK : last, g.K);
    stage_store<KA, kBM, SWZ>(ra[0], lds, sa);
    stage_store<KB, BN, SWZ>(rb[0], lds + kBufA, sb);
    __syncthreads();

    // step s: buffer s % 2 is multiplied, registers (s + 1) % 2 are decoded
    // into buffer (s + 1) % 2, registers s % 2 receive the loads of step s + 2
    auto step = [&](int64_t s, auto par) {
        constexpr int P = decltype(par)::value;
        const uint16_t* la = lds + P * (kBufA + kBufB);
        const uint16_t* lb = la + kBufA;
        uint16_t* wa = lds + (P ^ 1) * (kBufA + kBufB);
        uint16_t* wb = wa + kBufA;
        bf16x8_t fa[2][kTI], fb[2][TJ];
        load_frags<BN, SWZ>(la, lb, 0, fa[0], fb[0]);
        const int64_t kn = (s + 2) * kBK < last ? (s + 2) * kBK : last;
        stage_load<KA, kBM, FAST, FULL>(ra[P], g.a, m0, kn, g.K);
        stage_load<KB, BN, FAST, FULL>(rb[P], g.b, n0, kn, g.K);
        // keep the scheduler from sinking these loads towards their use in
        // the next step (which would shorten the prefetch to nothing)
        __builtin_amdgcn_sched_barrier(0);
        TBuf<kBM> ta;
        TBuf<BN> tb;
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            if (ks + 1 < kBK / 16) load_frags<BN, SWZ>(la, lb, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
            stage_store_part<KA, kBM, SWZ>(ra[P ^ 1], ta, wa, sa, ks);
            stage_store_part<KB, BN, SWZ>(rb[P ^ 1], tb, wb, sb, ks);
#pragma unroll
            for (int i = 0; i < kTI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][i], fb[ks & 1][j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    };
    for (int64_t s = 0; s < steps; s += 2) {
        step(s, std::integral_constant<int, 0>{});
        if (s + 1 < steps) step(s + 1, std::integral_constant<int, 1>{});
    }

    // accumulator e of lane l in MFMA tile (i, j): row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32
#pragma unroll
    for (int i = 0; i < kTI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int64_t col = n0 + wn * (BN / 2) + j * 32 + (l & 31);
            if (col >= g.N) continue;
            if constexpr (kTransposedOut<KA>) {
                // C stored transposed (element (row, col) at col * M + row; M
                // % 16 == 0): accumulators 4q .. 4q + 3 are four consecutive
                // rows, so one 8-byte store each
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t row = m0 + wm * 32 * kTI + i * 32 + 8 * q + 4 * (l >> 5);
                    if (row < g.M)
                        *reinterpret_cast<u32x2*>(g.c + col * g.M + row) =
                            u32x2{pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                  pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = m0 + wm * 32 * kTI + i * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
                    if (row < g.M) g.c[row * g.N + col] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.0f) & 0xFFFFu);
                }
            }
        }
}

int64_t tile_count(int64_t rows, int64_t cols, int bn) { return ((rows + kBM - 1) / kBM) * ((cols + bn - 1) / bn); }

// 256-wide tiles for the forward product (both operands NVFP4) when they
// give every compute unit of the chip (256 on MI355X) a tile, else 128-wide
// ones; the backward products (one bf16 operand, whose staging registers
// leave no room for 256-wide accumulators) always take 128-wide tiles
template <int KA, int KB>
hipError_t launch_gemm(const Operand& a, const Operand& b, uint16_t* c, int64_t M, int64_t N, int64_t K,
                       hipStream_t stream)
{
    GemmArgs g;
    g.a = a;
    g.b = b;
    g.c = c;
    g.M = M;
    g.N = N;
    g.K = K;
    constexpr bool kCanWiden = KA == OP_FP4_K && KB == OP_FP4_K;
    const bool wide = kCanWiden && tile_count(M, N, 256) >= 256;
    const int bn = wide ? 256 : 128;
    g.tiles_m = (int)((M + kBM - 1) / kBM);
    g.tiles_n = (int)((N + bn - 1) / bn);
    const dim3 grid((unsigned)tile_count(M, N, bn));
    // the vector load forms: NVFP4 operands stored [rows][K] need K % 32 ==
    // 0; a bf16 grad_y needs its row length N % 8 == 0 ([M][N] read along N)
    // or N % 4 == 0 (read along M)
    // (and with every tile inside: M % 256, N % BN, K % 64 all 0, no masks)
    const bool fast = KA == OP_FP4_K   ? (K % 32) == 0
                      : KA == OP_FP4_T ? (b.ld % 8) == 0   // B is grad_y read along N
                      : KA == OP_BF16_K ? (a.ld % 8) == 0
                                        : (a.ld % 4) == 0;
    const bool full = fast && M % kBM == 0 && N % bn == 0 && K % kBK == 0;
    const dim3 block(kThreads);
    if constexpr (kCanWiden) {
        if (wide) {
            if (full)
                hipLaunchKernelGGL((w4a4_gemm_kernel<KA, KB, 256, true, true>), grid, block, 0, stream, g);
            else if (fast)
                hipLaunchKernelGGL((w4a4_gemm_kernel<KA, KB, 256, true, false>), grid, block, 0, stream, g);
            else
                hipLaunchKernelGGL((w4a4_gemm_kernel<KA, KB, 256, false, false>), grid, block, 0, stream, g);
            return hipGetLastError();
        }
    }
    if (full)
        hipLaunchKernelGGL((w4a4_gemm_kernel<KA, KB, 128, true, true>), grid, block, 0, stream, g);
    else if (fast)
        hipLaunchKernelGGL((w4a4_gemm_kernel<KA, KB, 128, true, false>), grid, block, 0, stream, g);
    else
        hipLaunchKernelGGL((w4a4_gemm_kernel<KA, KB, 128, false, false>), grid, block, 0, stream, g);
    return hipGetLastError();
}

inline size_t round16(size_t n) { return (n + 15) & ~(size_t)15; }
inline size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// packed NVFP4 operand of R x C elements: codes, then scales, then the tensor scale
size_t packed_scales_offset(int64_t R, int64_t C) { return (size_t)R * C / 2; }
size_t packed_tscale_offset(int64_t R, int64_t C) { return round16((size_t)R * C / 2 + (size_t)R * C / 16); }

Operand packed_operand(const void* packed, int64_t R, int64_t C, int64_t rows)
{
    const uint8_t* p = static_cast<const uint8_t*>(packed);
    Operand o;
    o.data = p;
    o.scales = p + packed_scales_offset(R, C);
    o.tscale = reinterpret_cast<const float*>(p + packed_tscale_offset(R, C));
    o.ld = C;
    o.rows = rows;
    return o;
}

Operand bf16_operand(const void* data, int64_t ld, int64_t rows)
{
    Operand o;
    o.data = data;
    o.scales = nullptr;
    o.tscale = nullptr;
    o.ld = ld;
    o.rows = rows;
    return o;
}

int64_t tiles(int64_t rows, int64_t cols) { return tile_count(rows, cols, 128); }

bool dims_ok(int64_t M, int64_t N, int64_t K)
{
    // every offset fits comfortably in 64 bits, and the tile grid of each of
    // the three products (y [M][N], grad_x [M][K], grad_w [N][K]) in an int
    constexpr int64_t kMax = (int64_t)1 << 30, kGrid = 0x7FFFFFFF;
    return M >= 0 && N >= 0 && K >= 0 && M < kMax && N < kMax && K < kMax && (K == 0 || (M < ((int64_t)1 << 36) / K &&
           N < ((int64_t)1 << 36) / K)) && (N == 0 || M < ((int64_t)1 << 36) / N) && tiles(M, N) <= kGrid &&
           tiles(M, K) <= kGrid && tiles(N, K) <= kGrid;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

// quantize one [R][C] operand into its packed form
qad_status_t quantize_packed(const void* src, qad_dtype_t dt, int64_t R, int64_t C, const uint8_t* scales_in,
                             const float* tscale_in, void* packed, void* workspace, size_t ws_bytes,
                             qad_stream_t stream)
{
    uint8_t* p = static_cast<uint8_t*>(packed);
    return nvfp4_quantize(src, dt, 1, R, C, scales_in, tscale_in, p, p + packed_scales_offset(R, C),
                          reinterpret_cast<float*>(p + packed_tscale_offset(R, C)), nullptr, workspace, ws_bytes,
                          stream);
}

} // namespace

size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (!dims_ok(M, N, K) || K <= 0 || K % 16 != 0) return 0;   // the entry points' shape rule
    const size_t rx = qad_workspace_bytes(QAD_OP_QUANTIZE, 1, M, K);
    const size_t rw = qad_workspace_bytes(QAD_OP_QUANTIZE, 1, N, K);
    return round256(rx > rw ? rx : rw);
}

} // namespace qad

extern "C" {

size_t qad_nvfp4_packed_bytes(int64_t R, int64_t C)
{
    if (R < 0 || C < 0 || C % 16 != 0 || (C > 0 && R > ((int64_t)1 << 40) / C)) return 0;
    return qad::packed_tscale_offset(R, C) + 16;
}

qad_status_t qad_w4a4_linear_fwd(const void* x, const void* w, qad_dtype_t dt, int64_t M, int64_t N, int64_t K,
                                 const uint8_t* w_scales_in, const float* w_tscale_in, void* y, void* xq, void* wq,
                                 void* workspace, size_t ws_bytes, qad_stream_t stream)
{
    using namespace qad;
    if (dt != QAD_BF16 && dt != QAD_F32) return QAD_ERR_DTYPE;
    if (!dims_ok(M, N, K) || K <= 0 || K % 16 != 0) return QAD_ERR_SHAPE;
    // empty outputs (M == 0 or N == 0) may be NULL; the other packed operand
    // is still written
    if ((M > 0 && (!x || !xq)) || (N > 0 && (!w || !wq)) || (M > 0 && N > 0 && !y) ||
        (w_scales_in == nullptr) != (w_tscale_in == nullptr))
        return QAD_ERR_INVALID_ARG;
    if (M == 0 && N == 0) return QAD_OK;
    if ((M > 0 && (!aligned16(x) || !aligned16(xq))) || (N > 0 && (!aligned16(w) || !aligned16(wq))) ||
        (M > 0 && N > 0 && !aligned16(y)))
        return QAD_ERR_ALIGNMENT;
    const size_t es = dt == QAD_BF16 ? 2 : 4;
    const size_t bx = qad_nvfp4_packed_bytes(M, K), bw = qad_nvfp4_packed_bytes(N, K), by = (size_t)M * N * 2;
    if (overlap(y, by, xq, bx) || overlap(y, by, wq, bw) || overlap(xq, bx, wq, bw) ||
        overlap(x, (size_t)M * K * es, y, by) || overlap(w, (size_t)N * K * es, y, by) ||
        overlap(x, (size_t)M * K * es, xq, bx) || overlap(w, (size_t)N * K * es, wq, bw))
        return QAD_ERR_INVALID_ARG;
    if (!workspace || ws_bytes < linear_workspace_bytes(M, N, K)) return QAD_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return QAD_ERR_ALIGNMENT;
    if (M > 0) {
        const qad_status_t st = quantize_packed(x, dt, M, K, nullptr, nullptr, xq, workspace, ws_bytes, stream);
        if (st != QAD_OK) return st;
    }
    if (N > 0) {
        const qad_status_t st = quantize_packed(w, dt, N, K, w_scales_in, w_tscale_in, wq, workspace, ws_bytes, stream);
        if (st != QAD_OK) return st;
    }
    if (M == 0 || N == 0) return QAD_OK;
    const hipError_t e = launch_gemm<OP_FP4_K, OP_FP4_K>(packed_operand(xq, M, K, M), packed_operand(wq, N, K, N),
                                                         static_cast<uint16_t*>(y), M, N, K,
                                                         reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? QAD_OK : QAD_ERR_HIP;
}

qad_status_t qad_w4a4_linear_bwd(const void* grad_y, const void* xq, const void* wq, int64_t M, int64_t N, int64_t K,
                                 void* grad_x, void* grad_w, void* workspace, size_t ws_bytes, qad_stream_t stream)
{
    using namespace qad;
    (void)workspace;
    (void)ws_bytes;
    if (!dims_ok(M, N, K) || K <= 0 || K % 16 != 0) return QAD_ERR_SHAPE;
    if (!grad_x && !grad_w && (M > 0 || N > 0)) return QAD_ERR_INVALID_ARG;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (M == 0 || N == 0) {
        // an empty sum: the other gradient is all zeros (K is even)
        if (M == 0 && grad_w && N > 0)
            return launch_fill_u32(static_cast<uint32_t*>(grad_w), N * K / 2, 0u, s) == hipSuccess ? QAD_OK : QAD_ERR_HIP;
        if (N == 0 && grad_x && M > 0)
            return launch_fill_u32(static_cast<uint32_t*>(grad_x), M * K / 2, 0u, s) == hipSuccess ? QAD_OK : QAD_ERR_HIP;
        return QAD_OK;
    }
    if (!grad_y || (grad_x && !wq) || (grad_w && !xq)) return QAD_ERR_INVALID_ARG;
    if (!aligned16(grad_y) || (grad_x && !aligned16(grad_x)) || (grad_w && !aligned16(grad_w)) ||
        (xq && !aligned16(xq)) || (wq && !aligned16(wq)))
        return QAD_ERR_ALIGNMENT;
    const size_t gyb = (size_t)M * N * 2, gxb = (size_t)M * K * 2, gwb = (size_t)N * K * 2;
    if ((grad_x && overlap(grad_x, gxb, grad_y, gyb)) || (grad_w && overlap(grad_w, gwb, grad_y, gyb)) ||
        (grad_x && grad_w && overlap(grad_x, gxb, grad_w, gwb)) ||
        (grad_x && overlap(grad_x, gxb, wq, qad_nvfp4_packed_bytes(N, K))) ||
        (grad_w && overlap(grad_w, gwb, xq, qad_nvfp4_packed_bytes(M, K))))
        return QAD_ERR_INVALID_ARG;
    if (grad_x) {
        // grad_x[M][K] = sum_n grad_y[m][n] wq(n, k), computed as its transpose
        // [K][M]: A = wq stored [N][K] (output rows k), B = grad_y rows, C
        // written transposed into grad_x.  The bf16 grad_y is then the
        // 128-wide operand, read K / 256 times instead of K / 128 times (the
        // other way round: grad_y as A, 32 KiB per step and tile; 298 -> 223
        // us on 8192 x 2048 x 4096); grad_w measured slower transposed
        // (212 -> 228 us), so it keeps grad_y^T as its A operand.
        const hipError_t e = launch_gemm<OP_FP4_T, OP_BF16_K>(packed_operand(wq, N, K, K), bf16_operand(grad_y, N, M),
                                                              static_cast<uint16_t*>(grad_x), K, M, N, s);
        if (e != hipSuccess) return QAD_ERR_HIP;
    }
    if (grad_w) {
        // grad_w[N][K] = sum_m grad_y[m][n] xq(m, k): A = grad_y stored [M][N], B = xq stored [M][K]
        const hipError_t e = launch_gemm<OP_BF16_T, OP_FP4_T>(bf16_operand(grad_y, N, N), packed_operand(xq, M, K, K),
                                                              static_cast<uint16_t*>(grad_w), N, K, M, s);
        if (e != hipSuccess) return QAD_ERR_HIP;
    }
    return QAD_OK;
}

} // extern "C"
