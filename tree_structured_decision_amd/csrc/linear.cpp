// Dense projections of a hybrid block: y [M, N] = x [M, K] w[N, K]^T (or
// y += x w^T, the residual connection folded into the product) on the
// flattened stream, fp32 accumulation. Rows are tokens, so one product
// covers every branch and the shared prefix is projected once. These are
// plain GEMMs and go to hipBLASLt: in its column-major terms y^T = w x^T,
// i.e. D (N x M, ld N) = op(A) B with A = w stored K x N (ld K) and
// transposed, B = x stored K x M (ld K).
//
// Per device: one hipBLASLt handle and one workspace, created at the first
// call; per (M, N, K, dtype): the descriptors and the heuristic's first
// algorithm, kept for the life of the process.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "common.h"

namespace fork {
namespace {

constexpr size_t kLtWorkspace = 32u << 20;
constexpr int kMaxDevices = 64;

struct LtPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;
  size_t ws = 0;
};

struct LtDevice {
  hipblasLtHandle_t h = nullptr;
  void* ws = nullptr;
  std::map<std::tuple<int, int, int, int>, LtPlan> plans;
};

std::mutex g_lt_mu;
LtDevice g_lt[kMaxDevices];

#define LT_CHECK(expr)                                                              \
  do {                                                                              \
    hipblasStatus_t s_ = (expr);                                                    \
    if (s_ != HIPBLAS_STATUS_SUCCESS) return fail(FORK_E_HIP, "%s: hipblasLt status %d", #expr, (int)s_); \
  } while (0)

fork_status make_plan(LtDevice& d, int M, int N, int K, hipDataType ty, LtPlan& p) {
  LT_CHECK(hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F));
  const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  LT_CHECK(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)));
  LT_CHECK(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)));
  LT_CHECK(hipblasLtMatrixLayoutCreate(&p.la, ty, K, N, K));
  LT_CHECK(hipblasLtMatrixLayoutCreate(&p.lb, ty, K, M, K));
  LT_CHECK(hipblasLtMatrixLayoutCreate(&p.lc, ty, N, M, N));
  hipblasLtMatmulPreference_t pref;
  LT_CHECK(hipblasLtMatmulPreferenceCreate(&pref));
  const uint64_t wsmax = kLtWorkspace;
  LT_CHECK(hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsmax,
                                                 sizeof(wsmax)));
  hipblasLtMatmulHeuristicResult_t res[1];
  int n = 0;
  const hipblasStatus_t hs = hipblasLtMatmulAlgoGetHeuristic(d.h, p.desc, p.la, p.lb, p.lc, p.lc, pref, 1, res, &n);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (hs != HIPBLAS_STATUS_SUCCESS || n < 1)
    return fail(FORK_E_UNSUPPORTED, "hipblasLt has no algorithm for M=%d N=%d K=%d (status %d)", M, N, K, (int)hs);
  p.algo = res[0].algo;
  p.ws = res[0].workspaceSize;
  return FORK_OK;
}

}  // namespace

fork_status launch_linear(const void* x, const void* w, void* y, int M, int N, int K, int accumulate,
                          fork_dtype dt, hipStream_t stream) {
  int dev = 0;
  FORK_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(FORK_E_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lk(g_lt_mu);
  LtDevice& d = g_lt[dev];
  if (!d.h) {
    LT_CHECK(hipblasLtCreate(&d.h));
    FORK_HIP_CHECK(hipMalloc(&d.ws, kLtWorkspace));
  }
  const auto key = std::make_tuple(M, N, K, (int)dt);
  auto it = d.plans.find(key);
  if (it == d.plans.end()) {
    LtPlan p;
    const fork_status st = make_plan(d, M, N, K, dt == FORK_BF16 ? HIP_R_16BF : HIP_R_32F, p);
    if (st) return st;
    it = d.plans.emplace(key, p).first;
  }
  const LtPlan& p = it->second;
  const float alpha = 1.f, beta = accumulate ? 1.f : 0.f;
  LT_CHECK(hipblasLtMatmul(d.h, p.desc, &alpha, w, p.la, x, p.lb, &beta, y, p.lc, y, p.lc, &p.algo, d.ws, p.ws,
                           stream));
  return FORK_OK;
}

}  // namespace fork
