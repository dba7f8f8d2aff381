// Stand-ins for the kernel launchers, for a host-only build of the C ABI's
// argument checks (csrc/api.cpp with the host plans of csrc/plan.cpp) under
// the address and undefined-behaviour sanitizers, without a GPU compiler.
// Each launcher records what it was handed and returns success; nothing is
// computed and no device memory is touched.  Test infrastructure only.
#include <string.h>

#include "../../reduced_query_head_amd/csrc/launch.h"

namespace sqa {
namespace {
int g_kind = 0;   // 1 forward, 2 backward, 3 decode, 4 decode without workspace, 5 layer
LaunchArgs g_fwd;
BwdArgs g_bwd;
DecodeArgs g_dec;
LayerArgs g_layer;
}  // namespace

hipError_t launch_attn_fwd(const LaunchArgs& a) {
  g_kind = 1;
  g_fwd = a;
  return hipSuccess;
}
hipError_t launch_attn_bwd(const BwdArgs& a) {
  g_kind = 2;
  g_bwd = a;
  return hipSuccess;
}
hipError_t launch_attn_decode(const DecodeArgs& a) {
  g_kind = 3;
  g_dec = a;
  return hipSuccess;
}
hipError_t launch_attn_decode_noalloc(const DecodeArgs& a) {
  g_kind = 4;
  g_dec = a;
  return hipSuccess;
}
hipError_t launch_layer_fwd(const LayerArgs& a, bool* lib_error) {
  g_kind = 5;
  g_layer = a;
  if (lib_error) *lib_error = false;
  return hipSuccess;
}
}  // namespace sqa

// What the last launcher received: kind (0 = none since the last reset), the
// softmax exponent factor c, the negate flag, and for the forward the row
// strides of q and of k/v; for the decode, whether a workspace was passed.
extern "C" __attribute__((visibility("default"))) void sqa_stub_reset() { sqa::g_kind = 0; }
extern "C" __attribute__((visibility("default"))) int sqa_stub_last(float* c, int* negate, int64_t* q_stride,
                                                                    int64_t* kv_stride, int* has_workspace) {
  *c = 0.f;
  *negate = 0;
  *q_stride = *kv_stride = 0;
  *has_workspace = 0;
  switch (sqa::g_kind) {
    case 1:
      *c = sqa::g_fwd.c;
      *negate = sqa::g_fwd.negate_q;
      *q_stride = sqa::g_fwd.q_stride;
      *kv_stride = sqa::g_fwd.kv_stride;
      break;
    case 2:
      *c = sqa::g_bwd.c;
      *negate = sqa::g_bwd.negate_q;
      *has_workspace = sqa::g_bwd.workspace != nullptr;
      break;
    case 3:
    case 4:
      *c = sqa::g_dec.c;
      *negate = sqa::g_dec.negate_q;
      *has_workspace = sqa::g_dec.workspace != nullptr;
      break;
    case 5:
      *c = sqa::g_layer.c;
      *negate = sqa::g_layer.negate_q;
      *has_workspace = sqa::g_layer.workspace != nullptr;
      break;
  }
  return sqa::g_kind;
}
