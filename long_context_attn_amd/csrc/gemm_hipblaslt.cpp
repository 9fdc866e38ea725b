// bf16 projections of the Lightning Attention layer on hipBLASLt, the
// baseline the library's own GEMM kernel (gemm.hip) is timed against: the
// library GEMMs either side of the attention ("Diving into MiniMax01 405B
// MoE", section "Hybrid Modeling", Mechanism step 1: q, k, v and the gate
// are linear maps of the layer input; the output is mapped back to the hidden
// size).  SiLU (for q, k, v, Mechanism step 2) is applied by hipBLASLt's
// epilogue to the fp32 accumulators, so the attention kernels then run on
// activated q, k, v; the gate's sigmoid stays in the attention's epilogue.
//
// Row-major Y [rows][n] = act(X [rows][k] W [k][n]) is the column-major
// product Y^T = W^T X^T: A = W as an n x k matrix with leading dimension n,
// B = X as k x rows with leading dimension k, D = Y^T as n x rows with
// leading dimension n; no transposes.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "la_internal.h"

namespace la {

namespace {

// One hipBLASLt handle per device, created on first use and kept until the
// process ends.
hipblasLtHandle_t device_handle(hipError_t* err) {
    static std::mutex mu;
    static hipblasLtHandle_t handles[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (handles[dev] == nullptr && hipblasLtCreate(&handles[dev]) != HIPBLAS_STATUS_SUCCESS) {
        handles[dev] = nullptr;
        *err = hipErrorNotInitialized;
    }
    return handles[dev];
}

// A matmul description with its layouts, and the algorithm the heuristic
// chose for it: built once per (device, shape, activation, workspace size)
// and kept until the process ends.
struct Plan {
    hipblasLtMatmulDesc_t op = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
    hipblasLtMatmulAlgo_t algo{};
};

struct Key {
    int dev;
    int64_t rows;
    int n, k, act;
    size_t ws;
    bool operator<(const Key& o) const {
        return std::tie(dev, rows, n, k, act, ws) < std::tie(o.dev, o.rows, o.n, o.k, o.act, o.ws);
    }
};

// Builds the plan of one shape; false if hipBLASLt cannot run it.
bool build_plan(hipblasLtHandle_t h, int64_t rows, int n, int k, GemmAct act, size_t ws,
                Plan* p) {
    bool ok = hipblasLtMatmulDescCreate(&p->op, HIPBLAS_COMPUTE_32F, HIP_R_32F) ==
              HIPBLAS_STATUS_SUCCESS;
    const hipblasOperation_t nop = HIPBLAS_OP_N;
    hipblasLtEpilogue_t epi = HIPBLASLT_EPILOGUE_DEFAULT;
    if (act == GemmAct::silu) epi = HIPBLASLT_EPILOGUE_SWISH_EXT;
    ok = ok &&
         hipblasLtMatmulDescSetAttribute(p->op, HIPBLASLT_MATMUL_DESC_TRANSA, &nop, sizeof(nop)) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(p->op, HIPBLASLT_MATMUL_DESC_TRANSB, &nop, sizeof(nop)) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(p->op, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)) ==
             HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&p->a, HIP_R_16BF, n, k, n) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&p->b, HIP_R_16BF, k, rows, k) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&p->d, HIP_R_16BF, n, rows, n) == HIPBLAS_STATUS_SUCCESS;
    hipblasLtMatmulPreference_t pref = nullptr;
    ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
    const uint64_t max_ws = ws;
    ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                     &max_ws, sizeof(max_ws)) ==
                   HIPBLAS_STATUS_SUCCESS;
    hipblasLtMatmulHeuristicResult_t res[1];
    int found = 0;
    ok = ok &&
         hipblasLtMatmulAlgoGetHeuristic(h, p->op, p->a, p->b, p->d, p->d, pref, 1, res, &found) ==
             HIPBLAS_STATUS_SUCCESS &&
         found >= 1 && res[0].workspaceSize <= ws;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (ok) p->algo = res[0].algo;
    return ok;
}

}  // namespace

size_t gemm_workspace_bytes() { return (size_t)64 << 20; }

hipError_t gemm_bf16(const void* x, const void* w, void* y, int64_t rows, int n, int k, GemmAct act,
                     void* workspace, size_t workspace_bytes, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    hipError_t err = hipSuccess;
    hipblasLtHandle_t h = device_handle(&err);
    if (h == nullptr) return err != hipSuccess ? err : hipErrorNotInitialized;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    static std::mutex mu;
    static std::map<Key, Plan>* plans = new std::map<Key, Plan>();  // kept to process end
    const Key key{dev, rows, n, k, (int)act, workspace_bytes};
    Plan plan;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = plans->find(key);
        if (it == plans->end()) {
            Plan fresh;
            if (!build_plan(h, rows, n, k, act, workspace_bytes, &fresh)) return hipErrorNotSupported;
            it = plans->emplace(key, fresh).first;
        }
        plan = it->second;
    }
    const float alpha = 1.0f, beta = 0.0f;
    if (hipblasLtMatmul(h, plan.op, &alpha, w, plan.a, x, plan.b, &beta, y, plan.d, y, plan.d,
                        &plan.algo, workspace, workspace_bytes, st) != HIPBLAS_STATUS_SUCCESS)
        return hipErrorLaunchFailure;
    return hipGetLastError();
}

}  // namespace la
