// Full attention layer with decoupled head counts: the GQA explainer's
// PyTorch module (q/k/v projections, K/V shared by groups of query heads,
// scaled_dot_product_attention, output projection) with the query-head count
// free as in Sparse Query Attention, whose abstract puts the saving in the
// smaller number of query heads: fewer attention-score FLOPs and narrower
// query and output projections.
//
//   qkv  = x W_qkv^T      one GEMM, W_qkv = [W_q; W_k; W_v] ([(H_q+2H_kv) d, d_model])
//   attn = attention(q, k, v) read in place from the qkv rows (row stride (H_q+2H_kv) d)
//   out  = attn W_o^T     W_o: [d_model, H_q d]
//
// The two projections are plain dense GEMMs and run on hipBLASLt (bf16 in and
// out, fp32 accumulation); the attention is this library's kernel.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <tuple>

#include "launch.h"

namespace sqa {
namespace {

constexpr int64_t kGemmWorkspace = kLayerGemmWorkspace;   // bytes of workspace offered to hipBLASLt

struct GemmPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  hipblasLtMatmulAlgo_t algo;
  size_t ws = 0;
};

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<std::tuple<int, int64_t, int64_t, int64_t, int64_t>, GemmPlan> g_plans;

hipblasLtHandle_t handle_for(int dev) {
  auto it = g_handles.find(dev);
  if (it != g_handles.end()) return it->second;
  hipblasLtHandle_t h = nullptr;
  if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) return nullptr;
  g_handles[dev] = h;
  return h;
}

// Y[M, N] (row-major, leading dimension ldy) = X[M, K] (row-major) . W[N, K]^T
// (row-major, an nn.Linear weight).  In hipBLASLt's column-major terms:
// Y^T (N x M) = op_T(W^T stored K x N) . X^T (K x M).
bool plan_gemm(int dev, hipblasLtHandle_t h, int64_t M, int64_t N, int64_t K, int64_t ldy, GemmPlan** out) {
  const auto key = std::make_tuple(dev, M, N, K, ldy);
  auto it = g_plans.find(key);
  if (it != g_plans.end()) {
    *out = &it->second;
    return true;
  }
  GemmPlan pl;
  if (hipblasLtMatmulDescCreate(&pl.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return false;
  const int32_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  hipblasLtMatmulDescSetAttribute(pl.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT));
  hipblasLtMatmulDescSetAttribute(pl.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN));
  if (hipblasLtMatrixLayoutCreate(&pl.a, HIP_R_16BF, (uint64_t)K, (uint64_t)N, K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&pl.b, HIP_R_16BF, (uint64_t)K, (uint64_t)M, K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&pl.c, HIP_R_16BF, (uint64_t)N, (uint64_t)M, ldy) != HIPBLAS_STATUS_SUCCESS)
    return false;
  hipblasLtMatmulPreference_t pref = nullptr;
  if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return false;
  const uint64_t max_ws = (uint64_t)kGemmWorkspace;
  hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &max_ws, sizeof(max_ws));
  hipblasLtMatmulHeuristicResult_t res[1];
  int n_res = 0;
  const hipblasStatus_t st =
      hipblasLtMatmulAlgoGetHeuristic(h, pl.desc, pl.a, pl.b, pl.c, pl.c, pref, 1, res, &n_res);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (st != HIPBLAS_STATUS_SUCCESS || n_res < 1 || res[0].workspaceSize > (size_t)kGemmWorkspace) return false;
  pl.algo = res[0].algo;
  pl.ws = res[0].workspaceSize;
  auto ins = g_plans.emplace(key, pl);
  *out = &ins.first->second;
  return true;
}

bool gemm_nt(int dev, hipblasLtHandle_t h, hipStream_t stream, const void* X, const void* W, void* Y, int64_t M,
             int64_t N, int64_t K, int64_t ldy, void* ws) {
  GemmPlan* pl = nullptr;
  if (!plan_gemm(dev, h, M, N, K, ldy, &pl)) return false;
  const float alpha = 1.0f, beta = 0.0f;
  return hipblasLtMatmul(h, pl->desc, &alpha, W, pl->a, X, pl->b, &beta, Y, pl->c, Y, pl->c, &pl->algo, ws,
                         pl->ws, stream) == HIPBLAS_STATUS_SUCCESS;
}

}  // namespace

hipError_t launch_layer_fwd(const LayerArgs& a, bool* lib_error) {
  *lib_error = false;
  const LayerPlan lp = layer_plan(a.B, a.S, a.H_q, a.H_kv, a.d);
  char* ws = (char*)a.workspace;
  uint16_t* qkv = (uint16_t*)ws;
  uint16_t* attn = (uint16_t*)(ws + lp.qkv_bytes);
  void* gws = ws + lp.qkv_bytes + lp.attn_bytes;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int64_t M = a.B * a.S;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    hipblasLtHandle_t h = handle_for(dev);
    if (!h || !gemm_nt(dev, h, (hipStream_t)a.stream, a.x, a.w_qkv, qkv, M, lp.n_qkv, a.d_model, lp.n_qkv, gws)) {
      *lib_error = true;
      return hipErrorUnknown;
    }
  }
  LaunchArgs at;
  at.q = qkv;
  at.k = qkv + (int64_t)a.H_q * a.d;
  at.v = qkv + (int64_t)(a.H_q + a.H_kv) * a.d;
  at.out = attn;
  at.lse = nullptr;
  at.B = a.B;
  at.S = a.S;
  at.H_q = a.H_q;
  at.H_kv = a.H_kv;
  at.d = a.d;
  at.dtype = 0;
  at.c = a.c;
  at.negate_q = a.negate_q;
  at.causal = a.causal;
  at.stream = a.stream;
  at.q_stride = lp.n_qkv;
  at.kv_stride = lp.n_qkv;
  e = launch_attn_fwd(at);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    hipblasLtHandle_t h = handle_for(dev);
    if (!h || !gemm_nt(dev, h, (hipStream_t)a.stream, attn, a.w_o, a.out, M, a.d_model, (int64_t)a.H_q * a.d,
                       a.d_model, gws)) {
      *lib_error = true;
      return hipErrorUnknown;
    }
  }
  return hipGetLastError();
}

}  // namespace sqa
