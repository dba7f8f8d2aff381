// Internal interface between the C-ABI layer (api.cpp) and the kernels.
#ifndef SQA_LAUNCH_H
#define SQA_LAUNCH_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sqa {

// Work decomposition shared by the kernels and the host plans (plan.cpp).
constexpr int kFwdRows = 32;      // query positions per forward item (one wave)
constexpr int kBwdRows = 32;      // query rows (dq) or keys (dk/dv) per backward wave
constexpr int kBwdWaves = 4;      // waves of a dq workgroup (a dk/dv workgroup has twice as many)
constexpr int kDkdvChunk = 32;    // key blocks of one group an XCD takes in a row (long sequences)
constexpr int kDecodeBlk = 32;    // keys per decode block (one S^T MFMA tile)
constexpr int kDecodeWaves = 4;   // waves per decode split (one workgroup)
constexpr int kDecodeCUs = 256;   // compute units a shared-split decode plan fills (MI355X)
constexpr int64_t kLayerGemmWorkspace = (int64_t)32 << 20;   // bytes offered to the GEMM library

// rows padded to the backward's 64-row tiles
__host__ __device__ constexpr int64_t pad64(int64_t s) { return (s + 63) / 64 * 64; }

struct LaunchArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;      // optional row log-normaliser output, [B, S, H_q]
  int64_t B;
  int64_t S;
  int32_t H_q;
  int32_t H_kv;
  int32_t d;
  int dtype;       // 0 = bf16, 1 = fp32
  float c;         // |scale| * log2(e), or a tiny positive value when scale == 0
  bool negate_q;   // scale < 0
  int causal;
  void* stream;
  int64_t q_stride;   // elements between consecutive positions of q (bf16 path; H_q * d when dense)
  int64_t kv_stride;  // same for k and v (bf16 path; H_kv * d when dense)
};

hipError_t launch_attn_fwd(const LaunchArgs& a);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;   // bwd_workspace_bytes(B, S, H_q) bytes
  int64_t B;
  int64_t S;
  int32_t H_q;
  int32_t H_kv;
  int32_t d;
  int dtype;         // 0 = bf16, 1 = fp32
  float c;           // |scale| * log2(e), or a tiny positive value when scale == 0
  bool negate_q;     // scale < 0
  float scale;       // signed scale
  int causal;
  void* stream;
};

hipError_t launch_attn_bwd(const BwdArgs& a);
int64_t bwd_workspace_bytes(int64_t B, int64_t S, int32_t H_q);
// dk/dv grid size; *kb_chunk = key blocks per XCD chunk (0: no chunking)
int64_t dkdv_layout(int64_t n_groups, int64_t key_blocks, int* kb_chunk);
int64_t bwd_grid_size(int64_t B, int64_t S, int32_t H_q, int32_t H_kv);
int64_t fwd_grid_size(int64_t B, int64_t S, int32_t H_q, int32_t H_kv);

struct DecodeArgs {
  const void* q;          // [B, H_q, d]
  const void* k;          // [B, S_max, H_kv, d]
  const void* v;
  const int32_t* seqlens; // [B] device array, or null (= S_max)
  void* out;              // [B, H_q, d]
  float* lse;             // [B, H_q] or null
  void* workspace;        // decode_plan(...).workspace_bytes bytes
  int64_t B;
  int64_t S_max;
  int32_t H_q;
  int32_t H_kv;
  int32_t d;
  int dtype;              // 0 = bf16, 1 = fp32
  float c;                // |scale| * log2(e), or a tiny positive value when scale == 0
  bool negate_q;          // scale < 0
  void* stream;
};

struct DecodePlan {
  int head_blocks;        // ceil(R / 32)
  int n_splits;
  int split_len;          // keys per split (a multiple of kDecodeBlk)
  bool coop;              // the waves of a workgroup share one split (H_kv < kDecodeWaves)
  int64_t n_wgs;          // split workgroups
  int64_t part_o_bytes;
  int64_t workspace_bytes;
};

// max_workspace > 0 lengthens the splits (fewer partial results) until the
// workspace fits in that many bytes; workspace_bytes still exceeds it when
// even one split per head does not fit.
DecodePlan decode_plan(int64_t B, int64_t S_max, int32_t H_q, int32_t H_kv, int32_t d, int64_t max_workspace = 0);
hipError_t launch_attn_decode(const DecodeArgs& a);

// Bytes of the library's own fixed decode scratch (one array per GPU).
constexpr int64_t kDecodeScratchBytes = (int64_t)16 << 20;
// Decode with a.workspace ignored: the partial results go to that scratch
// array of the stream's GPU; splits are planned to fit it.
hipError_t launch_attn_decode_noalloc(const DecodeArgs& a);

struct LayerArgs {
  const void* x;        // [B, S, d_model] bf16
  const void* w_qkv;    // [(H_q + 2 H_kv) d, d_model] bf16
  const void* w_o;      // [d_model, H_q d] bf16
  void* out;            // [B, S, d_model] bf16
  void* workspace;      // layer_plan(...).workspace_bytes bytes
  int64_t B;
  int64_t S;
  int32_t d_model;
  int32_t H_q;
  int32_t H_kv;
  int32_t d;
  float c;              // |scale| * log2(e), or a tiny positive value when scale == 0
  bool negate_q;        // scale < 0
  int causal;
  void* stream;
};

struct LayerPlan {
  int64_t n_qkv;            // (H_q + 2 H_kv) d, the fused projection width
  int64_t qkv_bytes;        // projection output, 256-byte rounded
  int64_t attn_bytes;       // attention output, 256-byte rounded
  int64_t gemm_ws_bytes;    // workspace offered to the GEMM library
  int64_t workspace_bytes;
};

LayerPlan layer_plan(int64_t B, int64_t S, int32_t H_q, int32_t H_kv, int32_t d);
// lib_error is set when the GEMM library (not the HIP runtime) failed
hipError_t launch_layer_fwd(const LayerArgs& a, bool* lib_error);

}  // namespace sqa

#endif
