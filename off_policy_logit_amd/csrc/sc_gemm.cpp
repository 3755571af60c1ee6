// Plain library GEMMs of the LM-head backward (dHidden = dZ W, dW = dZ^T X),
// through hipBLASLt: bf16 operands, fp32 accumulation.  One hipBLASLt handle
// per device is created on first use and kept for the process.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <mutex>

#include "sc_internal.h"

namespace sc {
namespace {

hipblasLtHandle_t handle_for_current_device(hipError_t* herr) {
  static std::mutex mu;
  static hipblasLtHandle_t handles[64] = {};
  int dev = 0;
  *herr = hipGetDevice(&dev);
  if (*herr != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!handles[dev] && hipblasLtCreate(&handles[dev]) != HIPBLAS_STATUS_SUCCESS)
    handles[dev] = nullptr;
  return handles[dev];
}

}  // namespace

// D (column-major m x n, leading dimension ldd) = op(A) op(B) + beta D, with
// op(A) m x k and op(B) k x n; A and B bf16 column-major (transposed when ta /
// tb), D fp32 (d_bf16 = 0) or bf16.  Returns hipSuccess or an error.
hipError_t gemm_bf16(bool ta, bool tb, int64_t m, int64_t n, int64_t k, const void* A,
                     int64_t lda, const void* B, int64_t ldb, float beta, void* D,
                     int d_bf16, int64_t ldd, void* ws, size_t ws_bytes, hipStream_t s) {
  hipError_t herr = hipSuccess;
  hipblasLtHandle_t h = handle_for_current_device(&herr);
  if (!h) return herr != hipSuccess ? herr : hipErrorNotInitialized;
  const hipDataType dt = d_bf16 ? HIP_R_16BF : HIP_R_32F;
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  hipError_t out = hipErrorUnknown;
  do {
    if (hipblasLtMatmulDescCreate(&op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS)
      break;
    const hipblasOperation_t opa = ta ? HIPBLAS_OP_T : HIPBLAS_OP_N;
    const hipblasOperation_t opb = tb ? HIPBLAS_OP_T : HIPBLAS_OP_N;
    if (hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa)) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)) !=
            HIPBLAS_STATUS_SUCCESS)
      break;
    if (hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, ta ? k : m, ta ? m : k, lda) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, tb ? n : k, tb ? k : n, ldb) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&ld, dt, m, n, ldd) != HIPBLAS_STATUS_SUCCESS)
      break;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) break;
    const uint64_t wsb = ws_bytes;
    if (hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                              &wsb, sizeof(wsb)) != HIPBLAS_STATUS_SUCCESS)
      break;
    hipblasLtMatmulHeuristicResult_t res[1];
    int nres = 0;
    if (hipblasLtMatmulAlgoGetHeuristic(h, op, la, lb, ld, ld, pref, 1, res, &nres) !=
            HIPBLAS_STATUS_SUCCESS ||
        nres < 1)
      break;
    const float one = 1.f;
    if (hipblasLtMatmul(h, op, &one, A, la, B, lb, &beta, D, ld, D, ld, &res[0].algo, ws,
                        ws_bytes, s) != HIPBLAS_STATUS_SUCCESS)
      break;
    out = hipSuccess;
  } while (false);
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ld) hipblasLtMatrixLayoutDestroy(ld);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (op) hipblasLtMatmulDescDestroy(op);
  return out;
}

}  // namespace sc
