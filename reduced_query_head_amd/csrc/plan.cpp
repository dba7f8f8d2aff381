// Host-side work plans of the kernels: grid sizes, workspace sizes and the
// decode split plan.  Plain C++ with no device code, so the argument checks
// of the C ABI (api.cpp) can also be built and tested without a GPU
// compiler (host sanitizer builds).
#include <stdint.h>

#include "launch.h"

namespace sqa {

namespace {
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
}  // namespace

// Forward grid at its largest shape (4 items per workgroup).
int64_t fwd_grid_size(int64_t B, int64_t S, int32_t H_q, int32_t H_kv) {
  const int64_t R = H_q / H_kv;
  const int64_t items = R * ((S + kFwdRows - 1) / kFwdRows);
  return B * H_kv * ((items + 3) / 4);
}

// dk/dv grid: one workgroup per (group, key block), or, for sequences of at
// least 64 key blocks, 32-block chunks dealt to the 8 XCDs (the grid padded
// to whole rounds of 8 chunks).
int64_t dkdv_layout(int64_t n_groups, int64_t key_blocks, int* kb_chunk) {
  if (key_blocks < 2 * kDkdvChunk) {
    *kb_chunk = 0;
    return n_groups * key_blocks;
  }
  *kb_chunk = kDkdvChunk;
  const int64_t units = n_groups * ((key_blocks + kDkdvChunk - 1) / kDkdvChunk);
  return (units + 7) / 8 * 8 * kDkdvChunk;
}

int64_t bwd_workspace_bytes(int64_t B, int64_t S, int32_t H_q) { return 2 * B * (int64_t)H_q * pad64(S) * 4; }

int64_t bwd_grid_size(int64_t B, int64_t S, int32_t H_q, int32_t H_kv) {
  const int64_t items = (int64_t)(H_q / H_kv) * ((S + kBwdRows - 1) / kBwdRows);
  const int64_t a = B * H_kv * ((items + kBwdWaves - 1) / kBwdWaves);
  int kb_chunk;
  const int64_t b = dkdv_layout(B * H_kv, (S + kBwdWaves * kBwdRows - 1) / (kBwdWaves * kBwdRows), &kb_chunk);
  const int64_t c = (B * H_q * pad64(S) * 8 + 255) / 256;
  return a > b ? (a > c ? a : c) : (b > c ? b : c);
}

// Split plan, first per wave: about 8 waves per wave slot of the chip (8 per
// CU), so that the last round is a small part of the work even when many
// splits are empty (short caches).  Wave ranges shorter than 512 keys are
// lengthened towards 512 as long as at least 2 waves per slot remain: short
// ones spend a larger share of their time starting up (512 instead of 256
// made the 32/8 and 16/8 head configurations of a 4 x 128K cache 1-3 %
// faster).  Each wave has at least 64 keys, and at least 16 keys per query
// head it serves, so the fp32 partial results written per split stay a
// small share of the cache bytes it reads.  With fewer K/V heads than waves
// per workgroup (coop), a split is the range of kDecodeWaves waves (one
// workgroup, merged in LDS), so one partial result covers four waves' keys;
// there the plan is one workgroup per CU instead, each wave at least 64
// keys, with no floor per served head.  Against the per-wave rule (A/B, one
// box, mixed cache lengths): 4 x 128K MQA 8/1 42.5 -> 39.4 us, GQA 32/2
// 97.3 -> 87.1 us, 8 x 128K GQA 32/2 169.9 -> 141.2 us, 1 x 32K MQA 32/1
// 27.0 -> 13.1 us (128 workgroups instead of 16), MQA 32/1 at 4 x 128K
// unchanged; 16 x 16K GQA 32/2 lost 5 %.  With four or more K/V heads each
// wave is a split of its own and a workgroup's waves read neighbouring heads
// of the same positions (measured 7-11 % faster there than the cooperative
// splits, which read one head).
DecodePlan decode_plan(int64_t B, int64_t S_max, int32_t H_q, int32_t H_kv, int32_t d, int64_t max_workspace) {
  DecodePlan pl;
  const int64_t R = H_q / H_kv;
  pl.head_blocks = (int)((R + 31) / 32);
  const int64_t units = B * H_kv * pl.head_blocks;
  const int64_t target_waves = 8 * 8 * 256, floor_waves = 2 * 8 * 256;
  const int64_t heads_per_wave = R < 32 ? R : 32;
  int64_t len = units > 0 ? (S_max * units + target_waves - 1) / target_waves : S_max;
  if (len < 512 && units > 0) {
    const int64_t len_floor = S_max * units / floor_waves;  // keeps >= floor_waves waves
    len = len_floor < 512 ? (len_floor > len ? len_floor : len) : 512;
  }
  pl.coop = H_kv < kDecodeWaves;
  if (pl.coop && units > 0) {
    // shared splits: one workgroup per CU, each wave a quarter of its split
    len = (S_max * units + kDecodeCUs * kDecodeWaves - 1) / (kDecodeCUs * kDecodeWaves);
    if (len < 64) len = 64;
  } else {
    if (len < 64) len = 64;
    if (len < 16 * heads_per_wave) len = 16 * heads_per_wave;
  }
  len = (len + kDecodeBlk - 1) / kDecodeBlk * kDecodeBlk;
  if (pl.coop) len *= kDecodeWaves;   // keys per split
  // a workspace bound: at most max_workspace / (bytes per split of every
  // head) splits, so each split covers at least S_max / that many keys
  const int64_t per_split = B * H_q * (int64_t)(d + 2) * 4;
  if (max_workspace > 0 && per_split > 0 && S_max > 0) {
    const int64_t max_splits = max_workspace / per_split;
    if (max_splits >= 1) {
      int64_t fit = (S_max + max_splits - 1) / max_splits;
      fit = (fit + kDecodeBlk - 1) / kDecodeBlk * kDecodeBlk;
      if (fit > len) len = fit;
    }
  }
  pl.split_len = (int)len;
  pl.n_splits = (int)(S_max > 0 ? (S_max + len - 1) / len : 1);
  pl.part_o_bytes = B * H_q * (int64_t)pl.n_splits * d * 4;
  pl.workspace_bytes = pl.part_o_bytes + B * H_q * (int64_t)pl.n_splits * 2 * 4;
  pl.n_wgs = pl.coop ? units * pl.n_splits : (units * pl.n_splits + kDecodeWaves - 1) / kDecodeWaves;
  return pl;
}

// Layer workspace: the fused projection output and the attention output
// (each rounded to 256 bytes), then the GEMM library's workspace.
LayerPlan layer_plan(int64_t B, int64_t S, int32_t H_q, int32_t H_kv, int32_t d) {
  LayerPlan p;
  p.n_qkv = ((int64_t)H_q + 2 * (int64_t)H_kv) * d;
  p.qkv_bytes = round_up(B * S * p.n_qkv * 2, 256);
  p.attn_bytes = round_up(B * S * (int64_t)H_q * d * 2, 256);
  p.gemm_ws_bytes = kLayerGemmWorkspace;
  p.workspace_bytes = p.qkv_bytes + p.attn_bytes + p.gemm_ws_bytes;
  return p;
}

}  // namespace sqa
