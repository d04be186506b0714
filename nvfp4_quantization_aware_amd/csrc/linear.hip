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
// MFMA GEMM: each workgroup stages 128 x 64 tiles of both operands into LDS,
// rebuilding the QDQ values bf16(dec(code) * s_eff) there exactly as the
// quantizer's own bf16 output is formed (FP4 decode, one binary32 product,
// nearest-even bf16), then four waves multiply them with
// v_mfma_f32_32x32x16_bf16 into fp32 accumulators.  So the operands cross HBM
// as 4-bit codes, never as bf16 QDQ copies.
#include "libqad.h"

#include "qad_device.h"
#include "qad_internal.h"

namespace qad {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;   // workgroup tile
constexpr int kThreads = 256;                    // four waves, 2 x 2 over the tile
constexpr int kLds = kBK + 8;                    // LDS row stride in bf16 (144 B: conflict-free 16-B reads)

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
    int64_t M, N, K;        // K: contraction length (a multiple of 16)
    int tiles_m, tiles_n;
};

// Staging registers of one thread for one 128 x 64 tile of an operand.
//   *_K: row r = t / 2 of the tile, contraction [32 h, 32 h + 32), h = t % 2
//   *_T: contraction rows [8 kb, 8 kb + 8), kb = t / 32, output [4 o, 4 o + 4), o = t % 32
template <int KIND> struct Stage;
template <> struct Stage<OP_BF16_K> { u32x4 v[4]; };
template <> struct Stage<OP_FP4_K> { u32x2 code[2]; uint32_t sc; };
template <> struct Stage<OP_BF16_T> { u32x2 v[8]; };
template <> struct Stage<OP_FP4_T> { uint32_t code[4]; uint32_t sc[2]; };

__device__ __forceinline__ u32x4 ld16(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// Global loads of the tile whose output rows start at row0 and contraction at
// k0; what lies outside the operand reads as zeros (code 0 decodes to +0).
template <int KIND>
__device__ __forceinline__ void stage_load(Stage<KIND>& s, const Operand& op, int64_t row0, int64_t k0, int64_t K)
{
    const int t = threadIdx.x;
    if constexpr (KIND == OP_BF16_K || KIND == OP_FP4_K) {
        const int64_t row = row0 + (t >> 1);
        const int64_t kc = k0 + 32 * (t & 1);
        const bool rv = row < op.rows;
        if constexpr (KIND == OP_BF16_K) {
            const uint16_t* p = static_cast<const uint16_t*>(op.data) + row * op.ld + kc;
            const bool vec = (op.ld & 7) == 0;   // 16-byte aligned rows
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool ok = rv && kc + 8 * q < K;   // K % 16 == 0: a run of 8 lies wholly inside or outside
                if (ok && vec) {
                    s.v[q] = ld16(p + 8 * q);
                } else {
                    uint32_t w[4] = {0u, 0u, 0u, 0u};
                    if (ok)
                        for (int e = 0; e < 8; ++e) w[e >> 1] |= (uint32_t)p[8 * q + e] << (16 * (e & 1));
                    s.v[q] = u32x4{w[0], w[1], w[2], w[3]};
                }
            }
        } else {
            const uint8_t* codes = static_cast<const uint8_t*>(op.data) + row * (op.ld >> 1) + (kc >> 1);
            const uint8_t* sc = op.scales + row * (op.ld >> 4) + (kc >> 4);
            s.sc = 0u;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const bool ok = rv && kc + 16 * b < K;   // rows of whole blocks: 8-byte aligned
                s.code[b] = ok ? ld8(codes + 8 * b) : u32x2{0u, 0u};
                s.sc |= (ok ? (uint32_t)sc[b] : 0u) << (8 * b);
            }
        }
    } else {
        const int64_t kr0 = k0 + 8 * (t >> 5);
        const int64_t o = row0 + 4 * (t & 31);
        if constexpr (KIND == OP_BF16_T) {
            const bool vec = (op.ld & 3) == 0 && o + 4 <= op.rows;   // 8-byte aligned, wholly inside
#pragma unroll
            for (int i = 0; i < 8; ++i) {
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
            // four codes (2 bytes) and their block's scale per contraction row;
            // the output extent is a multiple of 16, so a run of 4 lies wholly
            // inside or outside
            const bool ov = o < op.rows;
            s.code[0] = s.code[1] = s.code[2] = s.code[3] = 0u;
            s.sc[0] = s.sc[1] = 0u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t kr = kr0 + i;
                const bool ok = ov && kr < K;
                const uint32_t c = ok ? *reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(op.data) +
                                                                           kr * (op.ld >> 1) + (o >> 1))
                                      : 0u;
                const uint32_t b = ok ? (uint32_t)op.scales[kr * (op.ld >> 4) + (o >> 4)] : 0u;
                s.code[i >> 1] |= c << (16 * (i & 1));
                s.sc[i >> 2] |= b << (8 * (i & 3));
            }
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

// Registers -> LDS tile [128 output rows][64 contraction] (bf16, stride kLds)
template <int KIND>
__device__ __forceinline__ void stage_store(const Stage<KIND>& s, uint16_t* lds, float s_g)
{
    const int t = threadIdx.x;
    if constexpr (KIND == OP_BF16_K || KIND == OP_FP4_K) {
        uint16_t* dst = lds + (t >> 1) * kLds + 32 * (t & 1);
        if constexpr (KIND == OP_BF16_K) {
#pragma unroll
            for (int q = 0; q < 4; ++q) lds_store16(dst + 8 * q, s.v[q]);
        } else {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const float se = e4m3_decode((s.sc >> (8 * b)) & 127u) * s_g;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t c = s.code[b][h];
                    lds_store16(dst + 16 * b + 8 * h,
                                u32x4{qdq_pair<0>(c, se), qdq_pair<1>(c, se), qdq_pair<2>(c, se), qdq_pair<3>(c, se)});
                }
            }
        }
    } else {
        // transpose: output row 4 o + e receives contraction [8 kb, 8 kb + 8)
        uint16_t* dst = lds + (4 * (t & 31)) * kLds + 8 * (t >> 5);
        uint32_t w[4][4];   // [e][pair of contraction rows]
        if constexpr (KIND == OP_BF16_T) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const u32x2 a = s.v[2 * p], b = s.v[2 * p + 1];
                w[0][p] = (a[0] & 0xFFFFu) | (b[0] << 16);
                w[1][p] = (a[0] >> 16) | (b[0] & 0xFFFF0000u);
                w[2][p] = (a[1] & 0xFFFFu) | (b[1] << 16);
                w[3][p] = (a[1] >> 16) | (b[1] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float v[2][4];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int i = 2 * p + r;
                    const float se = e4m3_decode((s.sc[i >> 2] >> (8 * (i & 3))) & 127u) * s_g;
                    const uint32_t c = s.code[i >> 1] >> (16 * (i & 1));
                    float lo, hi;
                    fp4_decode_pair<0>(c, lo, hi);
                    v[r][0] = lo * se;
                    v[r][1] = hi * se;
                    fp4_decode_pair<1>(c, lo, hi);
                    v[r][2] = lo * se;
                    v[r][3] = hi * se;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e][p] = pack_bf16x2(v[0][e], v[1][e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) lds_store16(dst + e * kLds, u32x4{w[e][0], w[e][1], w[e][2], w[e][3]});
    }
}

// tile index of workgroup `bid`: consecutive workgroups go to different XCDs
// (eight of them), so each XCD is given a contiguous run of tiles, ordered in
// groups of 8 tile rows so that a run shares operand tiles in its XCD's L2
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn)
{
    const int total = tiles_m * tiles_n;
    int id = bid;
    if ((total & 7) == 0) id = (bid & 7) * (total >> 3) + (bid >> 3);
    const int per_group = 8 * tiles_n;
    const int g = id / per_group, first = g * 8;
    const int gm = tiles_m - first < 8 ? tiles_m - first : 8;
    const int r = id - g * per_group;
    tm = first + r % gm;
    tn = r / gm;
}

// Operand loads run this many 64-deep steps ahead of the MFMAs: NVFP4 stages
// are 5 registers per operand, so three fit; bf16 stages are 16
template <int KA, int KB> struct Depth {
    static constexpr int value = (KA == OP_FP4_K || KA == OP_FP4_T) && (KB == OP_FP4_K || KB == OP_FP4_T) ? 3 : 1;
};

// One 64-deep step of the product: the registers of stage `st` are decoded
// into LDS, the loads of stage st + Depth are issued into the same
// registers, and the MFMAs consume the tile from LDS.
template <int KA, int KB>
__device__ __forceinline__ void gemm_step(const GemmArgs& g, Stage<KA>& ra, Stage<KB>& rb, int64_t st, int64_t steps,
                                          int64_t m0, int64_t n0, float sa, float sb, uint16_t* lds_a,
                                          uint16_t* lds_b, f32x16_t (&acc)[2][2])
{
    const int t = threadIdx.x, l = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    __syncthreads();   // the previous step's fragments have been read
    stage_store<KA>(ra, lds_a, sa);
    stage_store<KB>(rb, lds_b, sb);
    __syncthreads();
    constexpr int D = Depth<KA, KB>::value;
    if (st + D < steps) {
        stage_load<KA>(ra, g.a, m0, (st + D) * kBK, g.K);
        stage_load<KB>(rb, g.b, n0, (st + D) * kBK, g.K);
    }
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
        const int kcol = ks * 16 + 8 * (l >> 5);
        bf16x8_t fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            fa[i] = *reinterpret_cast<const bf16x8_t*>(lds_a + (wm * 64 + i * 32 + (l & 31)) * kLds + kcol);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            fb[j] = *reinterpret_cast<const bf16x8_t*>(lds_b + (wn * 64 + j * 32 + (l & 31)) * kLds + kcol);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
}

// C[M][N] = sum_k A(m, k) B(n, k), bf16 out of fp32 accumulation.  One
// 128 x 128 tile per workgroup; wave (wm, wn) owns the 64 x 64 quarter
// (wm, wn) as 2 x 2 MFMA tiles of 32 x 32.  Operand loads run Depth 64-deep
// steps ahead of the MFMAs, in a ring of register stages; each step decodes
// one stage into LDS.
template <int KA, int KB>
__global__ __launch_bounds__(kThreads) void w4a4_gemm_kernel(GemmArgs g)
{
    __shared__ __align__(16) uint16_t lds_a[kBM * kLds];
    __shared__ __align__(16) uint16_t lds_b[kBN * kLds];
    int tm, tn;
    tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int t = threadIdx.x, l = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const float sa = (KA == OP_FP4_K || KA == OP_FP4_T) ? *g.a.tscale : 0.0f;
    const float sb = (KB == OP_FP4_K || KB == OP_FP4_T) ? *g.b.tscale : 0.0f;

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

    const int64_t steps = (g.K + kBK - 1) / kBK;
    constexpr int D = Depth<KA, KB>::value;
    Stage<KA> ra[D];
    Stage<KB> rb[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d < steps) {
            stage_load<KA>(ra[d], g.a, m0, d * kBK, g.K);
            stage_load<KB>(rb[d], g.b, n0, d * kBK, g.K);
        }
    for (int64_t st = 0; st < steps; st += D) {
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (st + d < steps) gemm_step<KA, KB>(g, ra[d], rb[d], st + d, steps, m0, n0, sa, sb, lds_a, lds_b, acc);
    }

    // accumulator e of lane l in MFMA tile (i, j): row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + (l & 31);
            if (col >= g.N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
                if (row < g.M) g.c[row * g.N + col] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.0f) & 0xFFFFu);
            }
        }
}

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
    g.tiles_m = (int)((M + kBM - 1) / kBM);
    g.tiles_n = (int)((N + kBN - 1) / kBN);
    const int64_t tiles = (int64_t)g.tiles_m * g.tiles_n;
    hipLaunchKernelGGL((w4a4_gemm_kernel<KA, KB>), dim3((unsigned)tiles), dim3(kThreads), 0, stream, g);
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

int64_t tiles(int64_t rows, int64_t cols) { return ((rows + kBM - 1) / kBM) * ((cols + kBN - 1) / kBN); }

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
        // grad_x[M][K] = sum_n grad_y[m][n] wq(n, k): A = grad_y rows, B = wq stored [N][K]
        const hipError_t e = launch_gemm<OP_BF16_K, OP_FP4_T>(bf16_operand(grad_y, N, M), packed_operand(wq, N, K, K),
                                                              static_cast<uint16_t*>(grad_x), M, K, N, s);
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
