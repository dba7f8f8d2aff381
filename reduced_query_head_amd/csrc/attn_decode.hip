// Decode attention for gfx950 (MI355X, CDNA4): one new query token per
// sequence against that sequence's key/value cache.
//
//   out[b,h,:] = sum_{j < len_b} softmax_j(scale * <q[b,h,:], k[b,j,g,:]>) v[b,j,g,:],  g = floor(h / R)
//
// This is the regime the GQA explainer's background section describes: the
// whole cache (2 * H_kv * d values per position) is read for every generated
// token, so the kernel is bound by HBM bandwidth, and the K/V head count, not
// the query head count, sets its cost (the SQA abstract's contrast between
// this bandwidth-bound case and its compute-bound one).
//
// Split-KV design, two kernels:
//  * attn_decode_split: one wave per (b, K/V group g, block of up to 32 query
//    heads of the group, key split), four waves per workgroup.  The group's
//    query heads are the 32 columns of S^T = K Q^T on
//    v_mfma_f32_32x32x16_bf16 (keys along M), so a cache tile is read once
//    for all R heads that share it.  K comes straight from HBM into the
//    MFMA's A-operand registers; V goes global -> LDS by DMA into a
//    wave-private double buffer and is read back transposed
//    (ds_read_b64_tr_b16) for O^T += V^T P^T, as in the forward.  The waves
//    run their key loops independently (no barrier); K is loaded two blocks
//    ahead and V one block ahead, so each wave keeps about 24 KiB of cache
//    reads in flight.  Each split's running maximum m (log2 units), row sum
//    l and unnormalised O^T go to a workspace.  With fewer than four K/V
//    heads the four waves of a workgroup instead share one split, a quarter
//    of its keys each, and merge their results through LDS before writing
//    one partial result (a quarter of the partial traffic for MQA).
//  * attn_decode_combine: one workgroup per (b, h, 32 head dims) merges the
//    splits of that head: M = max m_s, L = sum l_s 2^(m_s - M),
//    O = sum O_s 2^(m_s - M) / L, and writes the bf16 output and
//    lse = ln2 (M + log2 L).
// Cache lengths come from a device array (or are all S_max); a length above
// S_max counts as S_max, and an empty cache gives out = 0, lse = -inf.
// fp32 inputs take the same plan and merge with the products on the fp32
// matrix cores (attn_decode_split_f32) and an fp32 output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace sqa {
namespace {

using namespace dev;

constexpr int kBlk = kDecodeBlk;  // keys per block (one S^T MFMA tile)
constexpr int kWavesDec = kDecodeWaves;   // waves per workgroup (one split)
constexpr float kLazyLog2D = 8.0f;

struct DecodeParams {
  const uint16_t* q;        // [B, H_q, D]
  const uint16_t* k;        // [B, S_max, H_kv, D]
  const uint16_t* v;
  const int32_t* seqlens;   // [B] or null
  float* part_o;            // [B, H_q, n_splits, D]
  float* part_ml;           // [B, H_q, n_splits, 2]
  uint16_t* out;            // [B, H_q, D]
  float* lse;               // [B, H_q] or null
  int S_max;
  int H_q;
  int H_kv;
  int R;
  int HB;                   // ceil(R / 32) query-head blocks per group
  int n_splits;
  int split_len;            // keys per split, multiple of kBlk
  float c;                  // |scale| * log2(e), > 0
  uint32_t q_sign;          // scale < 0: 0x8000 (bf16) or 0x80000000 (fp32), q negated on load (exact)
  int64_t n_waves;          // independent waves: B * H_kv * HB * n_splits
};

__device__ __forceinline__ int cache_len(const DecodeParams& p, int b) {
  const int len = p.seqlens ? p.seqlens[b] : p.S_max;
  return min(len, p.S_max);
}

// Merge of a shared split (COOP): waves 1-3 hand their running maxima, row
// sums and O^T to wave 0 through LDS (xo(w): wave w's O^T slot, DB*16*64
// floats); wave 0 rescales each to the larger maximum and adds it (an empty
// quarter holds m = -inf, l = 0, O = 0 and adds nothing; wave 0 always has
// keys).  Returns true in wave 0, which goes on to write the partial result.
template <int DB, class XO>
__device__ __forceinline__ bool coop_merge(f32x16 (&o)[DB], float& m_run, float& l_run, int wave, int lane, XO xo,
                                           float (*red_ml)[2][64]) {
  if (wave > 0) {
    SQA_LDS float* x = xo(wave);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[(db * 16 + r) * 64 + lane] = o[db][r];
    red_ml[wave][0][lane] = m_run;
    red_ml[wave][1][lane] = l_run;
  }
  __syncthreads();
  if (wave > 0) return false;
#pragma unroll
  for (int w = 1; w < kWavesDec; ++w) {
    const SQA_LDS float* x = xo(w);
    const float mw = red_ml[w][0][lane];
    const float m_new = fmaxf(m_run, mw);
    const float a0 = __builtin_amdgcn_exp2f(m_run - m_new);
    const float a1 = __builtin_amdgcn_exp2f(mw - m_new);
    l_run = l_run * a0 + red_ml[w][1][lane] * a1;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * a0 + x[(db * 16 + r) * 64 + lane] * a1;
      // keeps each wave's reads after the previous wave's sums
      asm volatile("" : "+v"(o[db]));
    }
    m_run = m_new;
  }
  return true;
}

template <int D, bool COOP>
__global__ __launch_bounds__(kWavesDec * 64, 2) void attn_decode_split_bf16(DecodeParams p) {
  constexpr int KS = D / 16;   // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;   // 32-dim blocks of O^T
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v[kWavesDec][2][kBlk * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // unit (b, split, head block, K/V head), K/V head fastest, so that units
  // that run together read all heads of the same cache positions (whole
  // rows).  Independent waves: one unit per wave.  COOP (fewer than four K/V
  // heads, where neighbouring units are other splits anyway): one unit per
  // workgroup, whose four waves take consecutive quarters of the split's
  // 32-key blocks and merge their partial results at the end, so that one
  // partial result covers four waves' keys.
  const int64_t uid = COOP ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * kWavesDec + wave;
  if (!COOP && uid >= p.n_waves) return;   // wave-uniform; no barrier on this path
  const int g = (int)(uid % p.H_kv);
  const int64_t r1 = uid / p.H_kv;
  const int hb = (int)(r1 % p.HB);
  const int64_t r2 = r1 / p.HB;
  const int split = (int)(r2 % p.n_splits);
  const int b = (int)(r2 / p.n_splits);

  const int len = cache_len(p, b);
  const int ks0 = split * p.split_len;
  if (ks0 >= len) return;         // empty split (uniform per unit): the combine step skips it
  const int ks1 = min(ks0 + p.split_len, len);
  // this wave's keys [k0, k1): the whole split, or its quarter (COOP; 0
  // blocks for an empty quarter of waves 1-3)
  const int q_blk = COOP ? ((ks1 - ks0 + kBlk - 1) / kBlk + kWavesDec - 1) / kWavesDec : 0;
  const int k0 = COOP ? ks0 + wave * q_blk * kBlk : ks0;
  const int k1 = COOP ? min(k0 + q_blk * kBlk, ks1) : ks1;
  const int n_blk = k1 > k0 ? (k1 - k0 + kBlk - 1) / kBlk : 0;

  const int hc = hb * 32 + col;   // query head of this lane's column, within the group
  const bool valid = hc < p.R;
  const int h = g * p.R + hc;

  const int64_t kv_stride = (int64_t)p.H_kv * D;
  const uint16_t* k_base = p.k + ((int64_t)b * p.S_max * p.H_kv + g) * D;
  const uint16_t* v_base = p.v + ((int64_t)b * p.S_max * p.H_kv + g) * D;

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  if (n_blk > 0) {
  TileCopy<D, 1, kBlk> cp;
  cp.init(kv_stride, 0, lane);
  SQA_LDS uint16_t* vbuf0 = (SQA_LDS uint16_t*)lds_v[wave][0];
  SQA_LDS uint16_t* vbuf1 = (SQA_LDS uint16_t*)lds_v[wave][1];
  cp.issue(v_base + (int64_t)k0 * kv_stride, kv_stride, k1 - k0, vbuf0, 0);

  // K rows as the A operand: lane holds key (row0 + col), head dims
  // ks*16 + half*8 ... +7; rows past the split end are clamped (and masked)
  bf16x8 kfa[KS], kfb[KS];   // K of even / odd blocks, loaded two blocks ahead
  auto load_k = [&](bf16x8 (&dst)[KS], int row0) {
    const int row = min(row0 + col, k1 - 1);
    const uint16_t* kp = k_base + (int64_t)row * kv_stride + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) dst[ks] = *(const bf16x8*)(kp + ks * 16);
  };
  // K loads are issued for every step, also past the split end (rows clamped
  // to the last valid one, cache hits): a fixed pattern of KS loads per step
  // that the wait counts below rely on
  load_k(kfa, k0);
  load_k(kfb, k0 + kBlk);

  // Q^T as the B operand: lane holds query head h (column col), same dims
  bf16x8 qf[KS];
  {
    const uint16_t* qp = p.q + ((int64_t)b * p.H_q + (valid ? h : g * p.R)) * D + half * 8;
    const uint32_t sgn = p.q_sign * 0x10001u;
    const uint32_t keep = valid ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = *(const u32x4*)(qp + ks * 16);
      raw ^= (u32x4){sgn, sgn, sgn, sgn};
      raw &= (u32x4){keep, keep, keep, keep};
      qf[ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // transposed V reads (same addressing as the forward's P.V step)
  int v_off[DB][2];
  {
    const int grp16 = lane >> 4, i16 = lane & 15, e = i16 >> 2, c4 = i16 & 3;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 2; ++j) v_off[db][j] = tile_off<D>(4 * half + 8 * j + e, db * 32 + (grp16 & 1) * 16 + 4 * c4);
  }

  const float c = p.c;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Block t needs V_t (copied in the previous step) and K_t (loaded two steps
  // earlier).  The only memory operations issued after both are the KS loads
  // of K_{t+1}: wait until at most those remain.
  auto step = [&](int t, bf16x8 (&kf)[KS], SQA_LDS uint16_t* vt, SQA_LDS uint16_t* vnext) {
    const int r0 = k0 + t * kBlk;
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KS) : "memory");

    // S^T = K Q^T: 32 keys x 32 query heads
    // V of the next block in flight first (its buffer held block t-1, whose
    // reads completed in the previous step), then K of the block after it
    if (t + 1 < n_blk) cp.issue(v_base + (int64_t)(r0 + kBlk) * kv_stride, kv_stride, k1 - r0 - kBlk, vnext, 0);
    f32x16 s = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
    load_k(kf, r0 + 2 * kBlk);
    // keys past the split end: s[r] holds key r0 + 8*(r/4) + 4*half + r%4
    if (r0 + kBlk > k1) {
      const int lim = k1 - 1 - r0 - 4 * half;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) > lim) s[r] = -__builtin_inff();
    }

    // online softmax in the exp2 domain, running maximum moved lazily
    float mx = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = wave_pair_max(mx);
    const float m_cand = mx * c;
    const bool grow = m_cand > m_run + kLazyLog2D;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? m_cand : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    const float neg_m = -m_run;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, neg_m));

    // O^T += V^T P^T, 16 keys per MFMA; the row sum adds the same bf16 P
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[st * 8 + e];
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        psum = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pb[e], pb[e + 1]}, ones, psum, false);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SQA_LDS bf16x4*)(vt + st * 16 * D + v_off[db][0]));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SQA_LDS bf16x4*)(vt + st * 16 * D + v_off[db][1]));
        const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
      }
    }
    l_run += psum;
  };
  for (int t = 0; t < n_blk; t += 2) {
    step(t, kfa, vbuf0, vbuf1);
    if (t + 1 < n_blk) step(t + 1, kfb, vbuf1, vbuf0);
  }
  wait_copies();   // no load outlives the loop
  }

  if constexpr (COOP) {
    static_assert(DB * 16 * 64 * 4 <= 2 * kBlk * D * 2, "O^T fits a wave's two V buffers");
    __shared__ float red_ml[kWavesDec][2][64];
    // wave w's O^T goes to its own, now idle, V buffers
    if (!coop_merge(o, m_run, l_run, wave, lane, [&](int w) { return (SQA_LDS float*)lds_v[w][0]; }, red_ml))
      return;
  }

  const float l_tot = wave_pair_sum(l_run);
  if (!valid) return;
  const int64_t part = ((int64_t)b * p.H_q + h) * p.n_splits + split;
  if (half == 0) *(float2*)(p.part_ml + part * 2) = make_float2(m_run, l_tot);
  float* po = p.part_o + part * D;
  // O^T[db] register r holds head dim db*32 + 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(f32x4*)(po + db * 32 + 8 * j + 4 * half) =
          (f32x4){o[db][4 * j], o[db][4 * j + 1], o[db][4 * j + 2], o[db][4 * j + 3]};
}

// fp32 split kernel: the bf16 kernel's split plan, unit mapping, softmax,
// merge and partial-result layout, with both products on
// v_mfma_f32_32x32x2_f32 (fp32 operands and sums).  S^T = K Q^T: lane
// (key, half) supplies K[key][8j + 4*half + e] for k-step 4j + e from a
// 16-byte load of its row, and the Q^T operand uses the same dim order.
// O^T += V^T P^T: score register r supplies the key pair
// 8*(r/4) + r%4 (+ 4 in the upper half), V^T comes straight from HBM (32
// consecutive floats of a row per half-wave).  The next block's K and V are
// loaded into registers while the current one is computed.
template <int D, bool COOP>
__global__ __launch_bounds__(kWavesDec * 64, 1) void attn_decode_split_f32(DecodeParams p) {
  constexpr int DB = D / 32;   // 32-dim blocks of O^T
  constexpr int NQ = D / 8;    // 16-byte groups per wave half of a row
  constexpr int NV = 16 * DB;  // V operands per block
  __shared__ float lds_x[COOP ? (kWavesDec - 1) * DB * 16 * 64 : 4];

  const float* qg = (const float*)p.q;
  const float* kg = (const float*)p.k;
  const float* vg = (const float*)p.v;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  const int64_t uid = COOP ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * kWavesDec + wave;
  if (!COOP && uid >= p.n_waves) return;   // wave-uniform; no barrier on this path
  const int g = (int)(uid % p.H_kv);
  const int64_t r1 = uid / p.H_kv;
  const int hb = (int)(r1 % p.HB);
  const int64_t r2 = r1 / p.HB;
  const int split = (int)(r2 % p.n_splits);
  const int b = (int)(r2 / p.n_splits);

  const int len = cache_len(p, b);
  const int ks0 = split * p.split_len;
  if (ks0 >= len) return;         // empty split (uniform per unit): the combine step skips it
  const int ks1 = min(ks0 + p.split_len, len);
  const int q_blk = COOP ? ((ks1 - ks0 + kBlk - 1) / kBlk + kWavesDec - 1) / kWavesDec : 0;
  const int k0 = COOP ? ks0 + wave * q_blk * kBlk : ks0;
  const int k1 = COOP ? min(k0 + q_blk * kBlk, ks1) : ks1;
  const int n_blk = k1 > k0 ? (k1 - k0 + kBlk - 1) / kBlk : 0;

  const int hc = hb * 32 + col;   // query head of this lane's column, within the group
  const bool valid = hc < p.R;
  const int h = g * p.R + hc;

  // Q^T operand: dims 8j + 4*half + e at qf[4j + e]; zero for columns past R
  float qf[4 * NQ];
  {
    const float* qp = qg + ((int64_t)b * p.H_q + (valid ? h : g * p.R)) * D + 4 * half;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const f32x4 x = *(const f32x4*)(qp + 8 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * j + e] = valid ? __uint_as_float(__float_as_uint(x[e]) ^ p.q_sign) : 0.f;
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  if (n_blk > 0) {
    const int64_t kv_stride = (int64_t)p.H_kv * D;
    const float* k_base = kg + ((int64_t)b * p.S_max * p.H_kv + g) * D;
    const float* v_base = vg + ((int64_t)b * p.S_max * p.H_kv + g) * D;
    const float c = p.c;
    // block at row0: K of key row0 + col (dims 8j + 4*half ...), V of the keys
    // of score register r at head dims db*32 + col; rows past k1 clamped
    // (their scores are masked)
    auto load = [&](f32x4 (&kd)[NQ], float (&vd)[NV], int row0) {
      const float* kp = k_base + (int64_t)min(row0 + col, k1 - 1) * kv_stride + 4 * half;
#pragma unroll
      for (int j = 0; j < NQ; ++j) kd[j] = *(const f32x4*)(kp + 8 * j);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float* vp = v_base + (int64_t)min(row0 + 8 * (r >> 2) + 4 * half + (r & 3), k1 - 1) * kv_stride + col;
#pragma unroll
        for (int db = 0; db < DB; ++db) vd[r * DB + db] = vp[db * 32];
      }
    };
    auto step = [&](int t, f32x4 (&kc)[NQ], float (&vc)[NV], f32x4 (&kn)[NQ], float (&vn)[NV]) {
      const int r0 = k0 + t * kBlk;
      if (t + 1 < n_blk) load(kn, vn, r0 + kBlk);
      f32x16 s = (f32x16){};
#pragma unroll
      for (int j = 0; j < NQ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(kc[j][e], qf[4 * j + e], s, 0, 0, 0);
      // keys past the split end: s[r] holds key r0 + 8*(r/4) + 4*half + r%4
      if (r0 + kBlk > k1) {
        const int lim = k1 - 1 - r0 - 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) > lim) s[r] = -__builtin_inff();
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = wave_pair_max(mx);
      const float m_cand = mx * c;
      const bool grow = m_cand > m_run + kLazyLog2D;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? m_cand : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
      const float neg_m = -m_run;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, neg_m));
        psum += s[r];
      }
      l_run += psum;
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vc[r * DB + db], s[r], o[db], 0, 0, 0);
    };
    f32x4 ka[NQ], kb[NQ];
    float va[NV], vb[NV];
    load(ka, va, k0);
    for (int t = 0; t < n_blk; t += 2) {
      step(t, ka, va, kb, vb);
      if (t + 1 < n_blk) step(t + 1, kb, vb, ka, va);
    }
  }

  if constexpr (COOP) {
    __shared__ float red_ml[kWavesDec][2][64];
    if (!coop_merge(o, m_run, l_run, wave, lane,
                    [&](int w) { return (SQA_LDS float*)lds_x + (w - 1) * DB * 16 * 64; }, red_ml))
      return;
  }

  const float l_tot = wave_pair_sum(l_run);
  if (!valid) return;
  const int64_t part = ((int64_t)b * p.H_q + h) * p.n_splits + split;
  if (half == 0) *(float2*)(p.part_ml + part * 2) = make_float2(m_run, l_tot);
  float* po = p.part_o + part * D;
  // O^T[db] register r holds head dim db*32 + 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(f32x4*)(po + db * 32 + 8 * j + 4 * half) =
          (f32x4){o[db][4 * j], o[db][4 * j + 1], o[db][4 * j + 2], o[db][4 * j + 3]};
}

// One workgroup per (b, h, 32-dim chunk): merge the non-empty splits of that
// head for 32 of its head dims.  The 256 threads form 32 split groups of 8
// lanes, each lane holding 4 head dims (16-byte loads).  One pass over the
// splits, each group with its own running maximum, then an LDS reduction
// over the groups (a separate maximum pass before the weighted sum made this
// kernel 0.2-0.3 us, about 5 %, slower).
template <int D, bool F32OUT>
__global__ __launch_bounds__(256) void attn_decode_combine(DecodeParams p) {
  constexpr int DC = D / 32;            // dim chunks per head
  constexpr int LANES = 8;              // lanes per split group
  constexpr int SG = 256 / LANES;       // split groups
  __shared__ float red_mg[SG];
  __shared__ float red_l[SG];
  __shared__ f32x4 red_o[SG][LANES];
  const int tid = threadIdx.x;
  const int grp = tid / LANES;
  const int dl = tid % LANES;
  const int64_t row = blockIdx.x / DC;      // b * H_q + h
  const int dc = blockIdx.x % DC;
  const int b = (int)(row / p.H_q);
  const int len = cache_len(p, b);
  uint16_t* op = p.out + row * D + dc * 32;             // bf16 output
  float* opf = (float*)p.out + row * D + dc * 32;       // fp32 output
  if (len <= 0) {   // uniform over the workgroup
    if (tid < 32) {
      if constexpr (F32OUT) opf[tid] = 0.f;
      else op[tid] = 0;
    }
    if (p.lse && dc == 0 && tid == 0) p.lse[row] = -__builtin_inff();
    return;
  }
  const int n_valid = (len + p.split_len - 1) / p.split_len;
  const float* ml = p.part_ml + row * p.n_splits * 2;
  const float* po = p.part_o + row * p.n_splits * D + dc * 32;

  // one pass: each split group keeps its own running maximum and rescales
  // its sums when it grows; the groups are then combined with their maxima
  float Mg = -__builtin_inff();
  float L = 0.f;
  f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = grp; s < n_valid; s += SG) {
    const float2 mls = *(const float2*)(ml + 2 * s);
    const f32x4 o = *(const f32x4*)(po + (int64_t)s * D + dl * 4);
    const float mn = fmaxf(Mg, mls.x);
    const float a = __builtin_amdgcn_exp2f(Mg - mn);
    const float w = __builtin_amdgcn_exp2f(mls.x - mn);
    L = L * a + w * mls.y;
    acc = acc * a + w * o;
    Mg = mn;
  }
  red_o[grp][dl] = acc;
  if (dl == 0) {
    red_l[grp] = L;
    red_mg[grp] = Mg;
  }
  __syncthreads();
  if (tid < LANES) {
    float M = -__builtin_inff();
#pragma unroll
    for (int g2 = 0; g2 < SG; ++g2) M = fmaxf(M, red_mg[g2]);
    float Lt = 0.f;
    f32x4 o = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g2 = 0; g2 < SG; ++g2) {
      const float wg = __builtin_amdgcn_exp2f(red_mg[g2] - M);
      Lt += wg * red_l[g2];
      o += wg * red_o[g2][tid];
    }
    const float inv = 1.0f / Lt;
    if constexpr (F32OUT) {
      *(f32x4*)(opf + tid * 4) = o * inv;
    } else {
      bf16x4 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = (__bf16)(o[e] * inv);
      *(bf16x4*)(op + tid * 4) = w4;
    }
    if (p.lse && dc == 0 && tid == 0) p.lse[row] = (M + log2f(Lt)) * 0.69314718055994531f;
  }
}

template <int D>
hipError_t launch_decode_t(const DecodeArgs& a, const DecodePlan& plan) {
  DecodeParams p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.seqlens = a.seqlens;
  p.part_o = (float*)a.workspace;
  p.part_ml = (float*)((char*)a.workspace + plan.part_o_bytes);
  p.out = (uint16_t*)a.out;
  p.lse = a.lse;
  p.S_max = (int)a.S_max;
  p.H_q = a.H_q;
  p.H_kv = a.H_kv;
  p.R = a.H_q / a.H_kv;
  p.HB = plan.head_blocks;
  p.n_splits = plan.n_splits;
  p.split_len = plan.split_len;
  p.c = a.c;
  p.q_sign = a.dtype == 1 ? (a.negate_q ? 0x80000000u : 0u) : (a.negate_q ? 0x8000u : 0u);
  p.n_waves = a.B * a.H_kv * plan.head_blocks * plan.n_splits;
  const dim3 grid((unsigned)plan.n_wgs), block(kWavesDec * 64);
  if (a.dtype == 1) {
    if (plan.coop)
      hipLaunchKernelGGL((attn_decode_split_f32<D, true>), grid, block, 0, (hipStream_t)a.stream, p);
    else
      hipLaunchKernelGGL((attn_decode_split_f32<D, false>), grid, block, 0, (hipStream_t)a.stream, p);
  } else {
    if (plan.coop)
      hipLaunchKernelGGL((attn_decode_split_bf16<D, true>), grid, block, 0, (hipStream_t)a.stream, p);
    else
      hipLaunchKernelGGL((attn_decode_split_bf16<D, false>), grid, block, 0, (hipStream_t)a.stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = a.B * a.H_q;
  if (a.dtype == 1)
    hipLaunchKernelGGL((attn_decode_combine<D, true>), dim3((unsigned)(rows * (D / 32))), dim3(256), 0,
                       (hipStream_t)a.stream, p);
  else
    hipLaunchKernelGGL((attn_decode_combine<D, false>), dim3((unsigned)(rows * (D / 32))), dim3(256), 0,
                       (hipStream_t)a.stream, p);
  return hipGetLastError();
}

}  // namespace

namespace {

hipError_t launch_decode_planned(const DecodeArgs& a, const DecodePlan& plan) {
  switch (a.d) {
    case 32: return launch_decode_t<32>(a, plan);
    case 64: return launch_decode_t<64>(a, plan);
    case 128: return launch_decode_t<128>(a, plan);
  }
  return hipErrorInvalidValue;
}

// The fixed scratch of the allocation-free decode: the split kernel's
// partial results, for callers that cannot allocate device memory.  The
// runtime gives each GPU its own copy when it loads this code object; host
// code reaches a GPU's copy only through the address hipGetSymbolAddress
// returns with that GPU current (the array's name is a host-side stand-in).
// Nothing in it has to start at zero: the split kernel writes every partial
// result the combine kernel reads.
__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `device`'s scratch array, looked up once per device.
hipError_t scratch_address(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[device].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[device].load(std::memory_order_acquire);
    if (!p) {
      int current = -1;
      hipError_t e = hipGetDevice(&current);
      if (e != hipSuccess) return e;
      if (current != device && (e = hipSetDevice(device)) != hipSuccess) return e;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      const hipError_t e2 = current != device ? hipSetDevice(current) : hipSuccess;
      if (e != hipSuccess) return e;
      if (e2 != hipSuccess) return e2;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[device].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_decode(const DecodeArgs& a) {
  return launch_decode_planned(a, decode_plan(a.B, a.S_max, a.H_q, a.H_kv, a.d));
}

hipError_t launch_attn_decode_noalloc(const DecodeArgs& a) {
  const DecodePlan plan = decode_plan(a.B, a.S_max, a.H_q, a.H_kv, a.d, kDecodeScratchBytes);
  if (plan.workspace_bytes > kDecodeScratchBytes) return hipErrorInvalidValue;
  DecodeArgs b = a;
  int device = -1;
  hipError_t e = a.stream ? hipStreamGetDevice((hipStream_t)a.stream, &device) : hipGetDevice(&device);
  if (e != hipSuccess) return e;
  if ((e = scratch_address(device, &b.workspace)) != hipSuccess) return e;
  return launch_decode_planned(b, plan);
}

}  // namespace sqa
