// bf16 projections of the Lightning Attention layer on hipBLASLt: the
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

#include <mutex>

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

struct Desc {
    hipblasLtMatmulDesc_t op = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
    hipblasLtMatmulPreference_t pref = nullptr;
    ~Desc() {
        if (pref) hipblasLtMatmulPreferenceDestroy(pref);
        if (d) hipblasLtMatrixLayoutDestroy(d);
        if (b) hipblasLtMatrixLayoutDestroy(b);
        if (a) hipblasLtMatrixLayoutDestroy(a);
        if (op) hipblasLtMatmulDescDestroy(op);
    }
};

}  // namespace

size_t gemm_workspace_bytes() { return (size_t)64 << 20; }

hipError_t gemm_bf16(const void* x, const void* w, void* y, int64_t rows, int n, int k, GemmAct act,
                     void* workspace, size_t workspace_bytes, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    hipError_t err = hipSuccess;
    hipblasLtHandle_t h = device_handle(&err);
    if (h == nullptr) return err != hipSuccess ? err : hipErrorNotInitialized;
    Desc dsc;
    bool ok = hipblasLtMatmulDescCreate(&dsc.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) ==
              HIPBLAS_STATUS_SUCCESS;
    const hipblasOperation_t nop = HIPBLAS_OP_N;
    hipblasLtEpilogue_t epi = HIPBLASLT_EPILOGUE_DEFAULT;
    if (act == GemmAct::silu) epi = HIPBLASLT_EPILOGUE_SWISH_EXT;
    ok = ok &&
         hipblasLtMatmulDescSetAttribute(dsc.op, HIPBLASLT_MATMUL_DESC_TRANSA, &nop, sizeof(nop)) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(dsc.op, HIPBLASLT_MATMUL_DESC_TRANSB, &nop, sizeof(nop)) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(dsc.op, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)) ==
             HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&dsc.a, HIP_R_16BF, n, k, n) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&dsc.b, HIP_R_16BF, k, rows, k) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&dsc.d, HIP_R_16BF, n, rows, n) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatmulPreferenceCreate(&dsc.pref) == HIPBLAS_STATUS_SUCCESS;
    const uint64_t max_ws = workspace_bytes;
    ok = ok && hipblasLtMatmulPreferenceSetAttribute(dsc.pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                     &max_ws, sizeof(max_ws)) ==
                   HIPBLAS_STATUS_SUCCESS;
    if (!ok) return hipErrorInvalidValue;
    hipblasLtMatmulHeuristicResult_t res[1];
    int found = 0;
    if (hipblasLtMatmulAlgoGetHeuristic(h, dsc.op, dsc.a, dsc.b, dsc.d, dsc.d, dsc.pref, 1, res,
                                        &found) != HIPBLAS_STATUS_SUCCESS ||
        found < 1 || res[0].workspaceSize > workspace_bytes)
        return hipErrorNotSupported;
    const float alpha = 1.0f, beta = 0.0f;
    if (hipblasLtMatmul(h, dsc.op, &alpha, w, dsc.a, x, dsc.b, &beta, y, dsc.d, y, dsc.d,
                        &res[0].algo, workspace, workspace_bytes, st) != HIPBLAS_STATUS_SUCCESS)
        return hipErrorLaunchFailure;
    return hipGetLastError();
}

}  // namespace la
