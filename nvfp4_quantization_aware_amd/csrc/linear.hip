// W4A4 NVFP4 fake-quant linear layer ([Qwen] "3. QAD": the student is the
// W4A4 NVFP4 model, weights and activations both NVFP4; [Lightning]
// "QAD的工作原理": simulated quantization runs in every student forward).
//
//   forward : y = QDQ(x) QDQ(w)^T        x [M][K], w [N][K], y [M][N]
//   backward: grad_x = grad_y QDQ(w),    grad_w = grad_y^T QDQ(x)
//             (straight-through through both quantizers)
//
// The two quantizers are the library's own one-HBM-pass QDQ kernels (dynamic
// per-tensor scales, blocks of 16 along K); their bf16 outputs xq, wq are
// returned for the backward.  The products are plain bf16 GEMMs with fp32
// accumulation on the MFMA units, through hipBLASLt.  Quantizing inside the
// GEMM's operand loads instead would repeat the ~12 VALU operations per
// element for every output tile that reloads the operand, which at
// 256-column tiles costs more VALU time than the element's MFMA work; one
// separate pass per operand costs one extra HBM round trip of it.
#include "libqad.h"

#include <hipblaslt/hipblaslt.h>
#include <map>
#include <mutex>
#include <tuple>

#include "qad_internal.h"

namespace {

constexpr size_t kGemmWorkspace = (size_t)64 << 20; // hipBLASLt scratch inside the caller's workspace

inline size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// one hipBLASLt handle per device, created on first use
hipblasLtHandle_t gemm_handle()
{
    static std::mutex mu;
    static hipblasLtHandle_t handles[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!handles[dev] && hipblasLtCreate(&handles[dev]) != HIPBLAS_STATUS_SUCCESS) handles[dev] = nullptr;
    return handles[dev];
}

// A prepared hipBLASLt product: descriptors and the chosen algorithm for one
// (device, transposes, m, n, k, leading dimensions), kept for reuse (a few
// hundred bytes each; building them and querying the heuristic costs far more
// host time than launching the product).
struct GemmPlan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
    hipblasLtMatmulAlgo_t algo{};
};

struct PlanKey {
    int dev;
    bool ta, tb;
    int64_t m, n, k, lda, ldb, ldd;
    bool operator<(const PlanKey& o) const
    {
        return std::tie(dev, ta, tb, m, n, k, lda, ldb, ldd) < std::tie(o.dev, o.ta, o.tb, o.m, o.n, o.k, o.lda, o.ldb, o.ldd);
    }
};

// The heuristic's candidates (up to kGemmCandidates) are timed on the first
// call's own operands and the fastest is kept: the heuristic's first choice
// runs some of these shapes at two thirds of the best candidate's rate.
// Timing synchronizes the stream once per plan; under graph capture (where
// that is not allowed) the first candidate is taken untimed.
constexpr int kGemmCandidates = 16;

bool make_plan(hipblasLtHandle_t h, const PlanKey& key, GemmPlan& p, const void* A, const void* B, void* D, void* ws,
               hipStream_t stream)
{
    if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return false;
    const int32_t opa = key.ta ? HIPBLAS_OP_T : HIPBLAS_OP_N, opb = key.tb ? HIPBLAS_OP_T : HIPBLAS_OP_N;
    if (hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa)) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)) != HIPBLAS_STATUS_SUCCESS)
        return false;
    // stored shapes (column-major rows x cols) before op
    if (hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, key.ta ? key.k : key.m, key.ta ? key.m : key.k, key.lda) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, key.tb ? key.n : key.k, key.tb ? key.k : key.n, key.ldb) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.ld, HIP_R_16BF, key.m, key.n, key.ldd) != HIPBLAS_STATUS_SUCCESS)
        return false;
    hipblasLtMatmulPreference_t pref = nullptr;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return false;
    const uint64_t wsb = kGemmWorkspace;
    hipblasLtMatmulHeuristicResult_t res[kGemmCandidates];
    int found = 0;
    const bool ok =
        hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb)) ==
            HIPBLAS_STATUS_SUCCESS &&
        hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.la, p.lb, p.ld, p.ld, pref, kGemmCandidates, res, &found) ==
            HIPBLAS_STATUS_SUCCESS &&
        found >= 1;
    hipblasLtMatmulPreferenceDestroy(pref);
    if (!ok) return false;
    p.algo = res[0].algo;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (found == 1 || hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return true;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess) return true;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return true;
    }
    const float alpha = 1.0f, beta = 0.0f;
    float best = 0.0f;
    for (int i = 0; i < found; ++i) {
        if (res[i].workspaceSize > kGemmWorkspace) continue;
        auto run = [&]() {
            return hipblasLtMatmul(h, p.desc, &alpha, A, p.la, B, p.lb, &beta, D, p.ld, D, p.ld, &res[i].algo, ws,
                                   kGemmWorkspace, stream) == HIPBLAS_STATUS_SUCCESS;
        };
        if (!run()) continue;   // warm-up (and a check that the candidate runs)
        bool good = hipEventRecord(e0, stream) == hipSuccess;
        for (int r = 0; r < 3 && good; ++r) good = run();
        good = good && hipEventRecord(e1, stream) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
        float ms = 0.0f;
        if (good && hipEventElapsedTime(&ms, e0, e1) == hipSuccess && (best == 0.0f || ms < best)) {
            best = ms;
            p.algo = res[i].algo;
        }
    }
    (void)hipEventDestroy(e1);
    (void)hipEventDestroy(e0);
    return true;
}

void free_plan(GemmPlan& p)
{
    if (p.ld) hipblasLtMatrixLayoutDestroy(p.ld);
    if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
    if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
    if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
}

// D (m x n, column-major, ld ldd) = op(A) op(B), bf16 operands and result,
// fp32 accumulation; A is m x k after op, B is k x n after op
qad_status_t gemm_bf16(bool ta, bool tb, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda, const void* B,
                       int64_t ldb, void* D, int64_t ldd, void* ws, hipStream_t stream)
{
    static std::mutex mu;
    static std::map<PlanKey, GemmPlan> plans;
    hipblasLtHandle_t h = gemm_handle();
    if (!h) return QAD_ERR_HIP;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QAD_ERR_HIP;
    const PlanKey key{dev, ta, tb, m, n, k, lda, ldb, ldd};
    GemmPlan plan;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = plans.find(key);
        if (it == plans.end()) {
            GemmPlan p;
            if (!make_plan(h, key, p, A, B, D, ws, stream)) {
                free_plan(p);
                return QAD_ERR_HIP;
            }
            it = plans.emplace(key, p).first;
        }
        plan = it->second;
    }
    const float alpha = 1.0f, beta = 0.0f;
    return hipblasLtMatmul(h, plan.desc, &alpha, A, plan.la, B, plan.lb, &beta, D, plan.ld, D, plan.ld, &plan.algo, ws,
                           kGemmWorkspace, stream) == HIPBLAS_STATUS_SUCCESS
               ? QAD_OK : QAD_ERR_HIP;
}

bool dims_ok(int64_t M, int64_t N, int64_t K)
{
    constexpr int64_t kMax = (int64_t)1 << 31;
    return M >= 0 && N >= 0 && K >= 0 && M < kMax && N < kMax && K < kMax && (K == 0 || (M < ((int64_t)1 << 36) / K &&
           N < ((int64_t)1 << 36) / K)) && (N == 0 || M < ((int64_t)1 << 36) / N);
}

bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

} // namespace

namespace qad {
size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    const size_t rx = qad_workspace_bytes(QAD_OP_QUANTIZE, 1, M, K);
    const size_t rw = qad_workspace_bytes(QAD_OP_QUANTIZE, 1, N, K);
    return round256(rx > rw ? rx : rw) + kGemmWorkspace;
}
} // namespace qad

extern "C" {

qad_status_t qad_w4a4_linear_fwd(const void* x, const void* w, qad_dtype_t dt, int64_t M, int64_t N, int64_t K,
                                 const uint8_t* w_scales_in, const float* w_tscale_in, void* y, void* xq, void* wq,
                                 void* workspace, size_t ws_bytes, qad_stream_t stream)
{
    if (dt != QAD_BF16 && dt != QAD_F32) return QAD_ERR_DTYPE;
    if (!dims_ok(M, N, K) || K <= 0 || K % 16 != 0) return QAD_ERR_SHAPE;
    // empty outputs (M == 0 or N == 0) may be NULL; the other QDQ output is
    // still written
    if ((M > 0 && (!x || !xq)) || (N > 0 && (!w || !wq)) || (M > 0 && N > 0 && !y) ||
        (w_scales_in == nullptr) != (w_tscale_in == nullptr))
        return QAD_ERR_INVALID_ARG;
    if (M == 0 && N == 0) return QAD_OK;
    if ((M > 0 && (!aligned16(x) || !aligned16(xq))) || (N > 0 && (!aligned16(w) || !aligned16(wq))) ||
        (M > 0 && N > 0 && !aligned16(y)))
        return QAD_ERR_ALIGNMENT;
    const size_t es = dt == QAD_BF16 ? 2 : 4;
    if (overlap(y, (size_t)M * N * 2, xq, (size_t)M * K * 2) || overlap(y, (size_t)M * N * 2, wq, (size_t)N * K * 2) ||
        overlap(xq, (size_t)M * K * 2, wq, (size_t)N * K * 2) || overlap(x, (size_t)M * K * es, y, (size_t)M * N * 2) ||
        overlap(w, (size_t)N * K * es, y, (size_t)M * N * 2))
        return QAD_ERR_INVALID_ARG;
    if (!workspace || ws_bytes < qad::linear_workspace_bytes(M, N, K)) return QAD_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return QAD_ERR_ALIGNMENT;
    const size_t rec = qad::linear_workspace_bytes(M, N, K) - kGemmWorkspace;
    if (M > 0) {
        const qad_status_t st = nvfp4_qdq_fwd(x, dt, 1, M, K, nullptr, nullptr, xq, workspace, rec, stream);
        if (st != QAD_OK) return st;
    }
    if (N > 0) {
        const qad_status_t st = nvfp4_qdq_fwd(w, dt, 1, N, K, w_scales_in, w_tscale_in, wq, workspace, rec, stream);
        if (st != QAD_OK) return st;
    }
    if (M == 0 || N == 0) return QAD_OK;
    // row-major y[M][N] = xq[M][K] wq[N][K]^T is the column-major N x M
    // product wq^T (K x N stored, transposed) times xq (K x M stored)
    return gemm_bf16(true, false, N, M, K, wq, K, xq, K, y, N, static_cast<char*>(workspace) + rec,
                     reinterpret_cast<hipStream_t>(stream));
}

qad_status_t qad_w4a4_linear_bwd(const void* grad_y, const void* xq, const void* wq, int64_t M, int64_t N, int64_t K,
                                 void* grad_x, void* grad_w, void* workspace, size_t ws_bytes, qad_stream_t stream)
{
    if (!dims_ok(M, N, K) || K <= 0 || K % 16 != 0) return QAD_ERR_SHAPE;
    if (!grad_x && !grad_w && (M > 0 || N > 0)) return QAD_ERR_INVALID_ARG;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (M == 0 || N == 0) {
        // an empty sum: the other gradient is all zeros (K is even)
        if (M == 0 && grad_w && N > 0) return qad::launch_fill_u32(static_cast<uint32_t*>(grad_w), N * K / 2, 0u, s) == hipSuccess ? QAD_OK : QAD_ERR_HIP;
        if (N == 0 && grad_x && M > 0) return qad::launch_fill_u32(static_cast<uint32_t*>(grad_x), M * K / 2, 0u, s) == hipSuccess ? QAD_OK : QAD_ERR_HIP;
        return QAD_OK;
    }
    if (!grad_y || (grad_x && !wq) || (grad_w && !xq)) return QAD_ERR_INVALID_ARG;
    if (!aligned16(grad_y) || (grad_x && !aligned16(grad_x)) || (grad_w && !aligned16(grad_w)) ||
        (xq && !aligned16(xq)) || (wq && !aligned16(wq)))
        return QAD_ERR_ALIGNMENT;
    if ((grad_x && overlap(grad_x, (size_t)M * K * 2, grad_y, (size_t)M * N * 2)) ||
        (grad_w && overlap(grad_w, (size_t)N * K * 2, grad_y, (size_t)M * N * 2)) ||
        (grad_x && grad_w && overlap(grad_x, (size_t)M * K * 2, grad_w, (size_t)N * K * 2)))
        return QAD_ERR_INVALID_ARG;
    if (!workspace || ws_bytes < qad::linear_workspace_bytes(M, N, K)) return QAD_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return QAD_ERR_ALIGNMENT;
    void* gws = static_cast<char*>(workspace) + (qad::linear_workspace_bytes(M, N, K) - kGemmWorkspace);
    if (grad_x) {
        // row-major grad_x[M][K] = grad_y[M][N] wq[N][K]: column-major K x M
        // = wq (K x N stored) times grad_y (N x M stored)
        qad_status_t st = gemm_bf16(false, false, K, M, N, wq, K, grad_y, N, grad_x, K, gws, s);
        if (st != QAD_OK) return st;
    }
    if (grad_w) {
        // row-major grad_w[N][K] = grad_y^T[N][M] xq[M][K]: column-major K x N
        // = xq (K x M stored) times grad_y^T (N x M stored, transposed)
        qad_status_t st = gemm_bf16(false, true, K, N, M, xq, K, grad_y, N, grad_w, K, gws, s);
        if (st != QAD_OK) return st;
    }
    return QAD_OK;
}

} // extern "C"
