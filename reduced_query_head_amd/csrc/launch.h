// Internal interface between the C-ABI layer (api.cpp) and the kernels.
#ifndef SQA_LAUNCH_H
#define SQA_LAUNCH_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sqa {

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
int64_t bwd_grid_size(int64_t B, int64_t S, int32_t H_q, int32_t H_kv);
int64_t bf16_grid_size(int64_t B, int64_t S, int32_t H_q, int32_t H_kv);

}  // namespace sqa

#endif
