// Prefill-sized products (batch above what the fused kernels take): the blob
// is decoded into a BF16 copy of W in the caller's workspace by the fused
// decode kernel, then one hipBLASLt GEMM multiplies it.  NWC describes its
// batched path the same way -- dequantize, then the vendor GEMM -- and says
// that it saves memory but no time ("NWC -- Neural Weight Compression", How
// it works, bullet "Dequantization and embedding lookup", and "Status and
// limitations"); Unweight's decompression into on-chip memory ahead of the
// matrix cores ("Unweight: how we compressed an LLM 22% without sacrificing
// quality", Direct GPU Decompression) is what the fused skinny kernel does
// for small batches instead.
//
// Row-major Y [batch][ldy] = X [batch][ldx] W'^T, W' [rows][ldw]: in the
// column-major terms of the BLAS, Y^T (rows x batch, ld ldy) = W' (as the
// transpose of a cols x rows matrix with ld ldw) times X^T (cols x batch,
// ld ldx), FP32 accumulation, D in BF16 or FP32.
#include <hip/hip_runtime_api.h>
#include <hipblaslt/hipblaslt.h>

#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "nwc_internal.hpp"

namespace {

constexpr size_t kBlasWorkspace = size_t{32} << 20;  // hipBLASLt's share of the workspace

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

// W' row stride: cols rounded up to 8 elements (16-byte rows for the decode)
uint64_t w_ld(uint64_t cols) { return (cols + 7) / 8 * 8; }

}  // namespace

// The caller's BLAS context: one hipBLASLt handle and the algorithm chosen
// for each problem shape seen so far (a heuristic query costs host time on
// every call otherwise).  Calls that share a context are serialised by its
// mutex for the cache lookup only.
struct nwc_blas {
  hipblasLtHandle_t handle = nullptr;
  std::mutex mu;
  using Key = std::tuple<uint64_t, uint64_t, uint64_t, uint64_t, uint64_t, uint64_t, int>;
  std::map<Key, hipblasLtMatmulAlgo_t> algos;
};

extern "C" {

nwc_status nwc_blas_create(nwc_blas** out) {
  if (!out) return NWC_ERR_INVALID_ARG;
  *out = nullptr;
  nwc_blas* h = new (std::nothrow) nwc_blas;
  if (!h) return NWC_ERR_HIP;
  if (hipblasLtCreate(&h->handle) != HIPBLAS_STATUS_SUCCESS) {
    delete h;
    return NWC_ERR_HIP;
  }
  *out = h;
  return NWC_OK;
}

nwc_status nwc_blas_destroy(nwc_blas* h) {
  if (!h) return NWC_ERR_INVALID_ARG;
  const bool ok = hipblasLtDestroy(h->handle) == HIPBLAS_STATUS_SUCCESS;
  delete h;
  return ok ? NWC_OK : NWC_ERR_HIP;
}

nwc_status nwc_prefill_workspace_size(const nwc_info* info, size_t* bytes) {
  nwc::Geometry g;
  if (!info || !bytes || !nwc::info_geometry(info, &g)) return NWC_ERR_INVALID_ARG;
  *bytes = up256(g.rows * w_ld(g.cols) * 2) + kBlasWorkspace;
  return NWC_OK;
}

nwc_status nwc_gemm_prefill(nwc_blas* h, const nwc_info* info, const void* blob_dev, const uint16_t* X_dev,
                            uint64_t ldx, int batch, void* Y_dev, uint64_t ldy, nwc_out_type y_type, void* ws,
                            size_t ws_bytes, void* stream) {
  nwc::Geometry g;
  if (!h || !info || !blob_dev || !X_dev || !Y_dev || !ws || batch < 1 || !nwc::info_geometry(info, &g))
    return NWC_ERR_INVALID_ARG;
  if (y_type != NWC_OUT_BF16 && y_type != NWC_OUT_F32) return NWC_ERR_INVALID_ARG;
  if (ldx < g.cols || ldy < g.rows) return NWC_ERR_INVALID_ARG;
  size_t need = 0;
  nwc_prefill_workspace_size(info, &need);
  if (ws_bytes < need) return NWC_ERR_BUFFER_TOO_SMALL;
  const uintptr_t xa = reinterpret_cast<uintptr_t>(X_dev), ya = reinterpret_cast<uintptr_t>(Y_dev),
                  wa = reinterpret_cast<uintptr_t>(ws);
  if ((xa & 15) || (ya & 15) || (wa & 255) || ldx % 8 || ldy % (y_type == NWC_OUT_F32 ? 4 : 8))
    return NWC_ERR_ALIGNMENT;
  const uint64_t ldw = w_ld(g.cols);
  uint16_t* w = static_cast<uint16_t*>(ws);
  void* blas_ws = static_cast<uint8_t*>(ws) + up256(g.rows * ldw * 2);

  // the decoded weights (validates the blob and its alignment)
  nwc_status st = nwc_decode(info, blob_dev, w, ldw, stream);
  if (st) return st;

  const hipDataType dt = y_type == NWC_OUT_F32 ? HIP_R_32F : HIP_R_16BF;
  const uint64_t m = g.rows, n = static_cast<uint64_t>(batch), k = g.cols;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  st = NWC_ERR_HIP;
  const hipblasOperation_t op_t = HIPBLAS_OP_T, op_n = HIPBLAS_OP_N;
  const uint64_t ws_cap = kBlasWorkspace;
  do {
    if (hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) break;
    if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &op_t, sizeof(op_t)) ||
        hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &op_n, sizeof(op_n)))
      break;
    if (hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, k, m, ldw) ||
        hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, k, n, ldx) ||
        hipblasLtMatrixLayoutCreate(&ld, dt, m, n, ldy))
      break;
    hipblasLtMatmulAlgo_t algo;
    bool have = false;
    const nwc_blas::Key key{m, n, k, ldw, ldx, ldy, static_cast<int>(dt)};
    {
      std::lock_guard<std::mutex> lock(h->mu);
      auto it = h->algos.find(key);
      if (it != h->algos.end()) {
        algo = it->second;
        have = true;
      }
    }
    if (!have) {
      if (hipblasLtMatmulPreferenceCreate(&pref) ||
          hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws_cap,
                                                sizeof(ws_cap)))
        break;
      hipblasLtMatmulHeuristicResult_t res[1];
      int found = 0;
      if (hipblasLtMatmulAlgoGetHeuristic(h->handle, desc, la, lb, ld, ld, pref, 1, res, &found) ||
          found < 1 || res[0].state != HIPBLAS_STATUS_SUCCESS) {
        st = NWC_ERR_UNSUPPORTED;
        break;
      }
      algo = res[0].algo;
      std::lock_guard<std::mutex> lock(h->mu);
      h->algos.emplace(key, algo);
    }
    const float alpha = 1.0f, beta = 0.0f;
    if (hipblasLtMatmul(h->handle, desc, &alpha, w, la, X_dev, lb, &beta, Y_dev, ld, Y_dev, ld, &algo, blas_ws,
                        kBlasWorkspace, static_cast<hipStream_t>(stream)) != HIPBLAS_STATUS_SUCCESS)
      break;
    st = NWC_OK;
  } while (false);
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ld) hipblasLtMatrixLayoutDestroy(ld);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (desc) hipblasLtMatmulDescDestroy(desc);
  return st;
}

}  // extern "C"
