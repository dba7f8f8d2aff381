// C-ABI entry points of libsqa: argument validation and kernel dispatch.
// Every check runs before any HIP call, so a rejected call has no effect.
#include <math.h>
#include <stdint.h>
#include <initializer_list>

#include "../../include/sqa.h"
#include "launch.h"

#define SQA_API extern "C" __attribute__((visibility("default")))

static_assert(sqa::kDecodeScratchBytes == SQA_DECODE_SCRATCH_BYTES, "scratch size differs from the header's");

namespace {

bool ranges_overlap(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// true when the product of the non-negative factors stays within int64
bool prod_ok(std::initializer_list<int64_t> factors) {
  int64_t x = 1;
  for (const int64_t f : factors)
    if (!mul_ok(x, f, &x)) return false;
  return true;
}

// Every product the decode split plan forms (keys x units, partial-result
// bytes, workgroups) is at most B * max(S_max, 1) * H_q * (d + 2) * 4.
bool decode_plan_fits(int64_t B, int64_t S_max, int32_t H_q, int32_t d) {
  return prod_ok({B, S_max > 0 ? S_max : 1, H_q, (int64_t)d + 2, 4});
}

// The backward's workspace and statistics grid are at most 8 * B * H_q * (S + 64).
bool bwd_plan_fits(int64_t B, int64_t S, int32_t H_q) {
  return S <= INT64_MAX - 64 && prod_ok({B, S + 64, H_q, 8});
}

// Kernels address a tile of up to 128 rows relative to a 64-bit tile base
// with 32-bit byte offsets: rows of up to 2^22 elements (32768 heads at
// d = 128) keep those under 1 GiB.
constexpr int64_t kMaxRowElems = (int64_t)1 << 22;

bool row_ok(int64_t heads, int32_t d) { return heads * d <= kMaxRowElems; }

}  // namespace

SQA_API const char* sqa_status_string(sqa_status status) {
  switch (status) {
    case SQA_OK: return "success";
    case SQA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SQA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SQA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

SQA_API sqa_status sqa_attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                                    int64_t B, int64_t S, int32_t H_q, int32_t H_kv, int32_t d,
                                    sqa_dtype dtype, float scale, int causal, sqa_stream_t stream) {
  // head counts: groups of H_q / H_kv query heads share one K/V head, so the
  // group count must divide the head count (GQA module's assertion)
  if (B < 0 || S < 0 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0) return SQA_ERR_INVALID_ARGUMENT;
  if (dtype != SQA_BF16 && dtype != SQA_FP32) return SQA_ERR_INVALID_ARGUMENT;
  if (causal != 0 && causal != 1) return SQA_ERR_INVALID_ARGUMENT;
  if (!isfinite(scale)) return SQA_ERR_INVALID_ARGUMENT;
  if (d < 1) return SQA_ERR_INVALID_ARGUMENT;
  if (B == 0 || S == 0) return SQA_OK;
  if (!q || !k || !v || !out) return SQA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u) return SQA_ERR_INVALID_ARGUMENT;

  const int64_t elem = dtype == SQA_BF16 ? 2 : 4;
  int64_t rows, q_elems, kv_elems, q_bytes, kv_bytes;
  if (!mul_ok(B, S, &rows) || !mul_ok(rows, (int64_t)H_q * d, &q_elems) ||
      !mul_ok(rows, (int64_t)H_kv * d, &kv_elems) || !mul_ok(q_elems, elem, &q_bytes) ||
      !mul_ok(kv_elems, elem, &kv_bytes))
    return SQA_ERR_INVALID_ARGUMENT;
  if (ranges_overlap(out, q_bytes, q, q_bytes) || ranges_overlap(out, q_bytes, k, kv_bytes) ||
      ranges_overlap(out, q_bytes, v, kv_bytes))
    return SQA_ERR_INVALID_ARGUMENT;
  if (lse) {
    int64_t lse_bytes;
    if (!mul_ok(rows, (int64_t)H_q * 4, &lse_bytes)) return SQA_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)lse & 3u) || ranges_overlap(lse, lse_bytes, q, q_bytes) ||
        ranges_overlap(lse, lse_bytes, k, kv_bytes) || ranges_overlap(lse, lse_bytes, v, kv_bytes) ||
        ranges_overlap(lse, lse_bytes, out, q_bytes))
      return SQA_ERR_INVALID_ARGUMENT;
  }

  if (d != 32 && d != 64 && d != 128) return SQA_ERR_UNSUPPORTED;
  if (!row_ok(H_q, d) || !row_ok(H_kv, d)) return SQA_ERR_UNSUPPORTED;
  // kernels index positions with 32-bit integers
  if (S > (int64_t)1 << 30) return SQA_ERR_UNSUPPORTED;
  // the bf16 and fp32 forward grids have at most fwd_grid_size workgroups
  if (sqa::fwd_grid_size(B, S, H_q, H_kv) > INT32_MAX) return SQA_ERR_UNSUPPORTED;

  sqa::LaunchArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.B = B;
  a.S = S;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.d = d;
  a.dtype = dtype == SQA_BF16 ? 0 : 1;
  // scores enter the softmax as scale * s * log2(e) so that exp2 can be used;
  // a negative scale is folded into q (exact for bf16: a sign flip)
  const float log2e = 1.4426950408889634f;
  const float mag = fabsf(scale);
  a.c = mag > 0.f ? mag * log2e : 1e-30f;
  if (!isfinite(a.c)) return SQA_ERR_INVALID_ARGUMENT;
  a.negate_q = scale < 0.f;
  a.causal = causal;
  a.stream = (void*)stream;
  a.q_stride = (int64_t)H_q * d;
  a.kv_stride = (int64_t)H_kv * d;
  return sqa::launch_attn_fwd(a) == hipSuccess ? SQA_OK : SQA_ERR_HIP;
}

SQA_API sqa_status sqa_attn_fwd(const void* q, const void* k, const void* v, void* out, int64_t B,
                                int64_t S, int32_t H_q, int32_t H_kv, int32_t d, sqa_dtype dtype,
                                float scale, int causal, sqa_stream_t stream) {
  return sqa_attn_fwd_lse(q, k, v, out, nullptr, B, S, H_q, H_kv, d, dtype, scale, causal, stream);
}

SQA_API int64_t sqa_attn_bwd_workspace_size(int64_t B, int64_t S, int32_t H_q) {
  if (B < 0 || S < 0 || H_q < 1 || !bwd_plan_fits(B, S, H_q)) return -1;
  return sqa::bwd_workspace_bytes(B, S, H_q);
}

SQA_API sqa_status sqa_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, void* workspace,
                                int64_t workspace_bytes, int64_t B, int64_t S, int32_t H_q, int32_t H_kv,
                                int32_t d, sqa_dtype dtype, float scale, int causal, sqa_stream_t stream) {
  if (B < 0 || S < 0 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0) return SQA_ERR_INVALID_ARGUMENT;
  if (dtype != SQA_BF16 && dtype != SQA_FP32) return SQA_ERR_INVALID_ARGUMENT;
  if (causal != 0 && causal != 1) return SQA_ERR_INVALID_ARGUMENT;
  if (!isfinite(scale) || d < 1) return SQA_ERR_INVALID_ARGUMENT;
  if (B == 0 || S == 0) return SQA_OK;
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || !workspace) return SQA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)workspace) & 15u)
    return SQA_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)lse & 3u) return SQA_ERR_INVALID_ARGUMENT;
  const int64_t elem = dtype == SQA_BF16 ? 2 : 4;
  int64_t rows, q_elems, kv_elems, q_bytes, kv_bytes, lse_bytes;
  if (!mul_ok(B, S, &rows) || !mul_ok(rows, (int64_t)H_q * d, &q_elems) ||
      !mul_ok(rows, (int64_t)H_kv * d, &kv_elems) || !mul_ok(q_elems, elem, &q_bytes) ||
      !mul_ok(kv_elems, elem, &kv_bytes) || !mul_ok(rows, (int64_t)H_q * 4, &lse_bytes))
    return SQA_ERR_INVALID_ARGUMENT;
  if (!bwd_plan_fits(B, S, H_q)) return SQA_ERR_UNSUPPORTED;
  const int64_t ws_need = sqa::bwd_workspace_bytes(B, S, H_q);
  if (workspace_bytes < ws_need) return SQA_ERR_INVALID_ARGUMENT;
  // outputs and workspace must not overlap each other or any input
  const void* ins[6] = {q, k, v, out, dout, lse};
  const int64_t in_bytes[6] = {q_bytes, kv_bytes, kv_bytes, q_bytes, q_bytes, lse_bytes};
  const void* outs[4] = {dq, dk, dv, workspace};
  const int64_t out_bytes[4] = {q_bytes, kv_bytes, kv_bytes, ws_need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (ranges_overlap(outs[i], out_bytes[i], ins[j], in_bytes[j])) return SQA_ERR_INVALID_ARGUMENT;
    for (int j = i + 1; j < 4; ++j)
      if (ranges_overlap(outs[i], out_bytes[i], outs[j], out_bytes[j])) return SQA_ERR_INVALID_ARGUMENT;
  }
  if (d != 32 && d != 64 && d != 128) return SQA_ERR_UNSUPPORTED;
  if (!row_ok(H_q, d) || !row_ok(H_kv, d)) return SQA_ERR_UNSUPPORTED;
  if (S > (int64_t)1 << 30) return SQA_ERR_UNSUPPORTED;
  // fp32: dq as the forward's grid, dk/dv one workgroup per 128 keys, the
  // statistics one thread per padded row
  if (dtype == SQA_BF16 ? sqa::bwd_grid_size(B, S, H_q, H_kv) > INT32_MAX
                        : (sqa::fwd_grid_size(B, S, H_q, H_kv) > INT32_MAX ||
                           (B * H_q * sqa::pad64(S) + 255) / 256 > INT32_MAX))
    return SQA_ERR_UNSUPPORTED;

  sqa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.workspace = workspace;
  a.B = B;
  a.S = S;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.d = d;
  a.dtype = dtype == SQA_BF16 ? 0 : 1;
  const float log2e = 1.4426950408889634f;
  const float mag = fabsf(scale);
  a.c = mag > 0.f ? mag * log2e : 1e-30f;
  if (!isfinite(a.c)) return SQA_ERR_INVALID_ARGUMENT;
  a.negate_q = scale < 0.f;
  a.scale = scale;
  a.causal = causal;
  a.stream = (void*)stream;
  return sqa::launch_attn_bwd(a) == hipSuccess ? SQA_OK : SQA_ERR_HIP;
}

SQA_API int64_t sqa_attn_decode_workspace_size(int64_t B, int64_t S_max, int32_t H_q, int32_t H_kv, int32_t d) {
  if (B < 0 || S_max < 0 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || d < 1) return -1;
  if (S_max > (int64_t)1 << 30 || B > ((int64_t)1 << 31) || !decode_plan_fits(B, S_max, H_q, d)) return -1;
  return sqa::decode_plan(B, S_max, H_q, H_kv, d).workspace_bytes;
}

namespace {

// Checks shared by both decode entry points; fills *a on success.  With
// no_alloc the partial results go to the library's fixed scratch instead of
// a caller workspace, so `workspace` must be null and the split plan must fit
// the scratch.
sqa_status decode_checks(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
                         void* out, float* lse, void* workspace, int64_t workspace_bytes, int64_t B,
                         int64_t S_max, int32_t H_q, int32_t H_kv, int32_t d, sqa_dtype dtype, float scale,
                         sqa_stream_t stream, bool no_alloc, sqa::DecodeArgs* a) {
  if (B < 0 || S_max < 0 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0) return SQA_ERR_INVALID_ARGUMENT;
  if (dtype != SQA_BF16 && dtype != SQA_FP32) return SQA_ERR_INVALID_ARGUMENT;
  if (!isfinite(scale) || d < 1) return SQA_ERR_INVALID_ARGUMENT;
  if (B == 0) return SQA_OK;
  if (!q || !out || (!no_alloc && !workspace) || (S_max > 0 && (!k_cache || !v_cache)))
    return SQA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out | (uintptr_t)workspace) & 15u)
    return SQA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)lse | (uintptr_t)seqlens) & 3u) return SQA_ERR_INVALID_ARGUMENT;
  if (S_max > (int64_t)1 << 30 || B > ((int64_t)1 << 31)) return SQA_ERR_UNSUPPORTED;
  const int64_t elem = dtype == SQA_BF16 ? 2 : 4;
  int64_t q_elems, q_bytes, cache_rows, kv_elems, kv_bytes, lse_bytes;
  if (!mul_ok(B, (int64_t)H_q * d, &q_elems) || !mul_ok(q_elems, elem, &q_bytes) ||
      !mul_ok(B, S_max, &cache_rows) || !mul_ok(cache_rows, (int64_t)H_kv * d, &kv_elems) ||
      !mul_ok(kv_elems, elem, &kv_bytes) || !mul_ok(B, (int64_t)H_q * 4, &lse_bytes))
    return SQA_ERR_INVALID_ARGUMENT;
  if (!decode_plan_fits(B, S_max, H_q, d)) return SQA_ERR_UNSUPPORTED;
  const sqa::DecodePlan plan =
      sqa::decode_plan(B, S_max, H_q, H_kv, d, no_alloc ? sqa::kDecodeScratchBytes : 0);
  if (!no_alloc && workspace_bytes < plan.workspace_bytes) return SQA_ERR_INVALID_ARGUMENT;
  const int64_t ws_bytes = no_alloc ? 0 : plan.workspace_bytes;
  const void* ins[4] = {q, k_cache, v_cache, seqlens};
  const int64_t in_bytes[4] = {q_bytes, kv_bytes, kv_bytes, seqlens ? B * 4 : 0};
  void* outs[3] = {out, lse, no_alloc ? nullptr : workspace};
  const int64_t out_bytes[3] = {q_bytes, lse ? lse_bytes : 0, ws_bytes};
  for (int i = 0; i < 3; ++i) {
    if (!outs[i]) continue;
    for (int j = 0; j < 4; ++j)
      if (ins[j] && ranges_overlap(outs[i], out_bytes[i], ins[j], in_bytes[j])) return SQA_ERR_INVALID_ARGUMENT;
    for (int j = i + 1; j < 3; ++j)
      if (outs[j] && ranges_overlap(outs[i], out_bytes[i], outs[j], out_bytes[j])) return SQA_ERR_INVALID_ARGUMENT;
  }
  if (d != 32 && d != 64 && d != 128) return SQA_ERR_UNSUPPORTED;
  if (!row_ok(H_q, d) || !row_ok(H_kv, d)) return SQA_ERR_UNSUPPORTED;
  // split grid (one workgroup per split or per four splits), combine grid (d/32 workgroups per row)
  if (plan.n_wgs > INT32_MAX || B * H_q * (d / 32) > INT32_MAX)
    return SQA_ERR_UNSUPPORTED;
  // the fixed scratch holds at least one split of every head
  if (no_alloc && plan.workspace_bytes > sqa::kDecodeScratchBytes) return SQA_ERR_UNSUPPORTED;

  a->q = q;
  a->k = k_cache;
  a->v = v_cache;
  a->seqlens = seqlens;
  a->out = out;
  a->lse = lse;
  a->workspace = no_alloc ? nullptr : workspace;
  a->B = B;
  a->S_max = S_max;
  a->H_q = H_q;
  a->H_kv = H_kv;
  a->d = d;
  a->dtype = dtype == SQA_BF16 ? 0 : 1;
  const float log2e = 1.4426950408889634f;
  const float mag = fabsf(scale);
  a->c = mag > 0.f ? mag * log2e : 1e-30f;
  if (!isfinite(a->c)) return SQA_ERR_INVALID_ARGUMENT;
  a->negate_q = scale < 0.f;
  a->stream = (void*)stream;
  return SQA_OK;
}

}  // namespace

SQA_API sqa_status sqa_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
                                   void* out, float* lse, void* workspace, int64_t workspace_bytes, int64_t B,
                                   int64_t S_max, int32_t H_q, int32_t H_kv, int32_t d, sqa_dtype dtype,
                                   float scale, sqa_stream_t stream) {
  sqa::DecodeArgs a;
  const sqa_status st = decode_checks(q, k_cache, v_cache, seqlens, out, lse, workspace, workspace_bytes, B, S_max,
                                      H_q, H_kv, d, dtype, scale, stream, false, &a);
  if (st != SQA_OK || B == 0) return st;
  return sqa::launch_attn_decode(a) == hipSuccess ? SQA_OK : SQA_ERR_HIP;
}

SQA_API sqa_status sqa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                           const int32_t* seqlens, void* out, float* lse, int64_t B, int64_t S_max,
                                           int32_t H_q, int32_t H_kv, int32_t d, sqa_dtype dtype, float scale,
                                           sqa_stream_t stream) {
  sqa::DecodeArgs a;
  const sqa_status st = decode_checks(q, k_cache, v_cache, seqlens, out, lse, nullptr, 0, B, S_max, H_q, H_kv, d,
                                      dtype, scale, stream, true, &a);
  if (st != SQA_OK || B == 0) return st;
  return sqa::launch_attn_decode_noalloc(a) == hipSuccess ? SQA_OK : SQA_ERR_HIP;
}

SQA_API int64_t sqa_layer_workspace_size(int64_t B, int64_t S, int32_t H_q, int32_t H_kv, int32_t d) {
  if (B < 0 || S < 0 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || d < 1) return -1;
  int64_t rows, t;
  if (!mul_ok(B, S, &rows) || !mul_ok(rows, ((int64_t)H_q + 2 * (int64_t)H_kv) * d * 4, &t)) return -1;
  return sqa::layer_plan(B, S, H_q, H_kv, d).workspace_bytes;
}

SQA_API sqa_status sqa_layer_fwd(const void* x, const void* w_qkv, const void* w_o, void* out, void* workspace,
                                 int64_t workspace_bytes, int64_t B, int64_t S, int32_t d_model, int32_t H_q,
                                 int32_t H_kv, int32_t d, float scale, int causal, sqa_stream_t stream) {
  if (B < 0 || S < 0 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || d < 1 || d_model < 1)
    return SQA_ERR_INVALID_ARGUMENT;
  if (causal != 0 && causal != 1) return SQA_ERR_INVALID_ARGUMENT;
  if (!isfinite(scale)) return SQA_ERR_INVALID_ARGUMENT;
  if (B == 0 || S == 0) return SQA_OK;
  if (!x || !w_qkv || !w_o || !out || !workspace) return SQA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)x | (uintptr_t)w_qkv | (uintptr_t)w_o | (uintptr_t)out | (uintptr_t)workspace) & 15u)
    return SQA_ERR_INVALID_ARGUMENT;
  int64_t rows, x_bytes, wqkv_bytes, wo_bytes, ws_probe;
  const int64_t n_qkv = ((int64_t)H_q + 2 * (int64_t)H_kv) * d;
  if (!mul_ok(B, S, &rows) || !mul_ok(rows, (int64_t)d_model * 2, &x_bytes) ||
      !mul_ok(n_qkv, (int64_t)d_model * 2, &wqkv_bytes) || !mul_ok((int64_t)H_q * d, (int64_t)d_model * 2, &wo_bytes) ||
      !mul_ok(rows, n_qkv * 4, &ws_probe))   // the workspace sizes stay representable
    return SQA_ERR_INVALID_ARGUMENT;
  const sqa::LayerPlan lp = sqa::layer_plan(B, S, H_q, H_kv, d);
  if (workspace_bytes < lp.workspace_bytes) return SQA_ERR_INVALID_ARGUMENT;
  const void* ins[3] = {x, w_qkv, w_o};
  const int64_t in_bytes[3] = {x_bytes, wqkv_bytes, wo_bytes};
  for (int j = 0; j < 3; ++j)
    if (ranges_overlap(out, x_bytes, ins[j], in_bytes[j]) ||
        ranges_overlap(workspace, lp.workspace_bytes, ins[j], in_bytes[j]))
      return SQA_ERR_INVALID_ARGUMENT;
  if (ranges_overlap(out, x_bytes, workspace, lp.workspace_bytes)) return SQA_ERR_INVALID_ARGUMENT;
  if (d != 32 && d != 64 && d != 128) return SQA_ERR_UNSUPPORTED;
  if (!row_ok((int64_t)H_q + 2 * (int64_t)H_kv, d)) return SQA_ERR_UNSUPPORTED;
  // rows of x, W_qkv and W_o must stay 16-byte aligned for the GEMM library
  if (d_model % 8 != 0) return SQA_ERR_UNSUPPORTED;
  if (S > (int64_t)1 << 30 || sqa::fwd_grid_size(B, S, H_q, H_kv) > INT32_MAX) return SQA_ERR_UNSUPPORTED;

  sqa::LayerArgs a;
  a.x = x;
  a.w_qkv = w_qkv;
  a.w_o = w_o;
  a.out = out;
  a.workspace = workspace;
  a.B = B;
  a.S = S;
  a.d_model = d_model;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.d = d;
  const float log2e = 1.4426950408889634f;
  const float mag = fabsf(scale);
  a.c = mag > 0.f ? mag * log2e : 1e-30f;
  if (!isfinite(a.c)) return SQA_ERR_INVALID_ARGUMENT;
  a.negate_q = scale < 0.f;
  a.causal = causal;
  a.stream = (void*)stream;
  bool lib_error = false;
  return sqa::launch_layer_fwd(a, &lib_error) == hipSuccess ? SQA_OK : SQA_ERR_HIP;
}
