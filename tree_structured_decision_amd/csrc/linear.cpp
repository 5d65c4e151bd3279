// Dense projections of a hybrid block: y [M, N] = x [M, K] w[N, K]^T (or
// y += x w^T, the residual connection folded into the product) on the
// flattened stream, fp32 accumulation. Rows are tokens, so one product
// covers every branch and the shared prefix is projected once. These are
// plain GEMMs and go to hipBLASLt: in its column-major terms y^T = w x^T,
// i.e. D (N x M, ld N) = op(A) B with A = w stored K x N (ld K) and
// transposed, B = x stored K x M (ld K).
//
// FP8 projections take E4M3 operands with one fp32 scale per row of each
// operand (per token of x, per output channel of w; device vectors, so
// scales computed on the GPU are used without a host round trip) and write
// bf16: y[m][n] = (sum_k xq[m][k] wq[n][k]) * x_scale[m] * w_scale[n]. In
// hipBLASLt's terms these are the outer-vector scales of A (w, N entries)
// and B (x, M entries).
//
// Per device: one hipBLASLt handle and one workspace, created at the first
// call; per (M, N, K, dtype): the descriptors and an algorithm, kept for the
// life of the process. The algorithm is the fastest of the heuristic's
// candidates, each timed once at that first call on the caller's operands
// (into a scratch output; the call synchronises the stream then).
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

// ty: the input type; the output has type oty. fp8 inputs carry per-tensor
// scale pointers (set on the descriptor before each product).
struct TuneArgs {
  const void* x;
  const void* w;
};
constexpr int kCandidates = 16;
constexpr int kTuneReps = 5;

fork_status make_plan(LtDevice& d, int M, int N, int K, hipDataType ty, hipDataType oty, LtPlan& p,
                      const TuneArgs* tune, hipStream_t stream, const float* a_scale = nullptr,
                      const float* b_scale = nullptr) {
  LT_CHECK(hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F));
  const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  LT_CHECK(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)));
  LT_CHECK(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)));
  LT_CHECK(hipblasLtMatrixLayoutCreate(&p.la, ty, K, N, K));
  LT_CHECK(hipblasLtMatrixLayoutCreate(&p.lb, ty, K, M, K));
  LT_CHECK(hipblasLtMatrixLayoutCreate(&p.lc, oty, N, M, N));
  if (a_scale) {
    const hipblasLtMatmulMatrixScale_t vec = HIPBLASLT_MATMUL_MATRIX_SCALE_OUTER_VEC_32F;
    LT_CHECK(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_A_SCALE_MODE, &vec, sizeof(vec)));
    LT_CHECK(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_B_SCALE_MODE, &vec, sizeof(vec)));
    LT_CHECK(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_A_SCALE_POINTER, &a_scale, sizeof(a_scale)));
    LT_CHECK(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_B_SCALE_POINTER, &b_scale, sizeof(b_scale)));
  }
  hipblasLtMatmulPreference_t pref;
  LT_CHECK(hipblasLtMatmulPreferenceCreate(&pref));
  const uint64_t wsmax = kLtWorkspace;
  LT_CHECK(hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsmax,
                                                 sizeof(wsmax)));
  hipblasLtMatmulHeuristicResult_t res[kCandidates];
  int n = 0;
  const hipblasStatus_t hs =
      hipblasLtMatmulAlgoGetHeuristic(d.h, p.desc, p.la, p.lb, p.lc, p.lc, pref, kCandidates, res, &n);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (hs != HIPBLAS_STATUS_SUCCESS || n < 1)
    return fail(FORK_E_UNSUPPORTED, "hipblasLt has no algorithm for M=%d N=%d K=%d (status %d)", M, N, K, (int)hs);
  p.algo = res[0].algo;
  p.ws = res[0].workspaceSize;
  if (n == 1 || !tune) return FORK_OK;
  // time the candidates once on the caller's operands (into a scratch output,
  // so the caller's y is untouched) and keep the fastest
  void* tmp = nullptr;
  const size_t ybytes = (size_t)M * N * (oty == HIP_R_32F ? 4 : 2);
  FORK_HIP_CHECK(hipMalloc(&tmp, ybytes));
  hipEvent_t e0, e1;
  FORK_HIP_CHECK(hipEventCreate(&e0));
  FORK_HIP_CHECK(hipEventCreate(&e1));
  const float alpha = 1.f, beta = 0.f;
  float best = 1e30f;
  for (int i = 0; i < n; ++i) {
    if (res[i].state != HIPBLAS_STATUS_SUCCESS || res[i].workspaceSize > kLtWorkspace) continue;
    bool ok = true;
    for (int r = 0; r < 2 + kTuneReps && ok; ++r) {
      if (r == 2) hipEventRecord(e0, stream);
      ok = hipblasLtMatmul(d.h, p.desc, &alpha, tune->w, p.la, tune->x, p.lb, &beta, tmp, p.lc, tmp, p.lc,
                           &res[i].algo, d.ws, res[i].workspaceSize, stream) == HIPBLAS_STATUS_SUCCESS;
    }
    if (!ok) continue;
    hipEventRecord(e1, stream);
    hipEventSynchronize(e1);
    float ms = 0.f;
    hipEventElapsedTime(&ms, e0, e1);
    if (ms < best) {
      best = ms;
      p.algo = res[i].algo;
      p.ws = res[i].workspaceSize;
    }
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  FORK_HIP_CHECK(hipStreamSynchronize(stream));
  FORK_HIP_CHECK(hipFree(tmp));
  return FORK_OK;
}

fork_status device_state(LtDevice** out) {
  int dev = 0;
  FORK_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(FORK_E_UNSUPPORTED, "device %d", dev);
  LtDevice& d = g_lt[dev];
  if (!d.h) {
    LT_CHECK(hipblasLtCreate(&d.h));
    FORK_HIP_CHECK(hipMalloc(&d.ws, kLtWorkspace));
  }
  *out = &d;
  return FORK_OK;
}

}  // namespace

fork_status launch_linear(const void* x, const void* w, void* y, int M, int N, int K, int accumulate,
                          fork_dtype dt, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_lt_mu);
  LtDevice* dp = nullptr;
  fork_status st = device_state(&dp);
  if (st) return st;
  LtDevice& d = *dp;
  const auto key = std::make_tuple(M, N, K, (int)dt);
  auto it = d.plans.find(key);
  if (it == d.plans.end()) {
    LtPlan p;
    const hipDataType ty = dt == FORK_BF16 ? HIP_R_16BF : HIP_R_32F;
    const TuneArgs ta{x, w};
    st = make_plan(d, M, N, K, ty, ty, p, &ta, stream);
    if (st) return st;
    it = d.plans.emplace(key, p).first;
  }
  const LtPlan& p = it->second;
  const float alpha = 1.f, beta = accumulate ? 1.f : 0.f;
  LT_CHECK(hipblasLtMatmul(d.h, p.desc, &alpha, w, p.la, x, p.lb, &beta, y, p.lc, y, p.lc, &p.algo, d.ws, p.ws,
                           stream));
  return FORK_OK;
}

fork_status launch_linear_fp8(const void* xq, const float* x_scale, const void* wq, const float* w_scale, void* y,
                              int M, int N, int K, int accumulate, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_lt_mu);
  LtDevice* dp = nullptr;
  fork_status st = device_state(&dp);
  if (st) return st;
  LtDevice& d = *dp;
  const auto key = std::make_tuple(M, N, K, 8);
  auto it = d.plans.find(key);
  if (it == d.plans.end()) {
    LtPlan p;
    const TuneArgs ta{xq, wq};
    st = make_plan(d, M, N, K, HIP_R_8F_E4M3, HIP_R_16BF, p, &ta, stream, w_scale, x_scale);
    if (st) return st;
    it = d.plans.emplace(key, p).first;
  }
  const LtPlan& p = it->second;
  // A is w, B is x in the column-major terms above
  LT_CHECK(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_A_SCALE_POINTER, &w_scale, sizeof(w_scale)));
  LT_CHECK(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_B_SCALE_POINTER, &x_scale, sizeof(x_scale)));
  const float alpha = 1.f, beta = accumulate ? 1.f : 0.f;
  LT_CHECK(hipblasLtMatmul(d.h, p.desc, &alpha, wq, p.la, xq, p.lb, &beta, y, p.lc, y, p.lc, &p.algo, d.ws, p.ws,
                           stream));
  return FORK_OK;
}

}  // namespace fork
