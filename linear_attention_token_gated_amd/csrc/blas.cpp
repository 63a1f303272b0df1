// blas.cpp -- the layer's plain projections (in-projection, gate, gates a|b,
// out-projection) through hipBLASLt.  They are ordinary dense products with
// no fused work, so the library's tuned gfx950 kernels serve them; everything
// specific to the method stays in this library's own kernels.
//
// C[M, N] = A[M, K] B[N, K]^T, all row-major, bf16 operands, fp32 accumulate,
// fp32 or bf16 C.  hipBLASLt is column-major, so the product is issued as
// C^T = B A^T: its "A" is B (K x N, leading dimension ldb, transposed), its
// "B" is A (K x M, leading dimension lda), its C is C^T (N x M, ldc).
//
// One handle per device, created on first use; per shape the descriptors and
// the algorithm chosen by the library's heuristic are kept for the life of
// the process.  No workspace is used, so a call allocates nothing.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "launch.hpp"

namespace gdn {

namespace {

struct Plan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    bool ok = false;
};

using Key = std::tuple<int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, bool>;

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<Key, Plan> g_plans;

// the plan for one shape on the current device; plan.ok is false when the
// library offers no algorithm for it
const Plan *plan_for(int dev, hipblasLtHandle_t h, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                     int64_t ldc, bool out_bf16)
{
    const Key key{dev, M, N, K, lda, ldb, ldc, out_bf16};
    auto it = g_plans.find(key);
    if (it != g_plans.end()) return &it->second;
    Plan pl;
    const int32_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    bool ok = hipblasLtMatmulDescCreate(&pl.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(pl.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(pl.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&pl.la, HIP_R_16BF, (uint64_t)K, (uint64_t)N, ldb) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&pl.lb, HIP_R_16BF, (uint64_t)K, (uint64_t)M, lda) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&pl.lc, out_bf16 ? HIP_R_16BF : HIP_R_32F, (uint64_t)N, (uint64_t)M, ldc) ==
                  HIPBLAS_STATUS_SUCCESS;
    if (ok) {
        hipblasLtMatmulPreference_t pref = nullptr;
        uint64_t ws = 0;
        hipblasLtMatmulHeuristicResult_t res[1];
        int nres = 0;
        ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
             hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof ws) ==
                 HIPBLAS_STATUS_SUCCESS &&
             hipblasLtMatmulAlgoGetHeuristic(h, pl.desc, pl.la, pl.lb, pl.lc, pl.lc, pref, 1, res, &nres) ==
                 HIPBLAS_STATUS_SUCCESS &&
             nres > 0 && res[0].state == HIPBLAS_STATUS_SUCCESS;
        if (ok) pl.algo = res[0].algo;
        if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    }
    pl.ok = ok;
    return &g_plans.emplace(key, pl).first->second;
}

}  // namespace

hipError_t blas_gemm_nt(const void *A, const void *B, void *C, bool out_bf16, int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc, hipStream_t stream)
{
    if (M == 0 || N == 0) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    hipblasLtHandle_t h = nullptr;
    const Plan *pl = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_handles.find(dev);
        if (it == g_handles.end()) {
            if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) return hipErrorNotSupported;
            g_handles.emplace(dev, h);
        } else {
            h = it->second;
        }
        pl = plan_for(dev, h, M, N, K, lda, ldb, ldc, out_bf16);
    }
    if (!pl->ok) return hipErrorNotSupported;
    const float alpha = 1.f, beta = 0.f;
    const hipblasStatus_t st = hipblasLtMatmul(h, pl->desc, &alpha, B, pl->la, A, pl->lb, &beta, C, pl->lc, C, pl->lc,
                                               &pl->algo, nullptr, 0, stream);
    return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace gdn
