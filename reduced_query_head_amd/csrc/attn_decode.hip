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
//    heads of the group, key split).  The group's query heads are the 32
//    columns of S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys along M), so a
//    cache tile is read once for all R heads that share it.  K comes straight
//    from HBM into the MFMA's A-operand registers; V goes global -> LDS by
//    DMA into a wave-private double buffer and is read back transposed
//    (ds_read_b64_tr_b16) for O^T += V^T P^T, as in the forward.  Waves are
//    independent (no workgroup barrier).  K is loaded two blocks ahead and V
//    one block ahead, so each wave keeps about 24 KiB of cache reads in
//    flight.  Each writes the split's running maximum m (log2 units), row sum
//    l and unnormalised O^T to a workspace.
//  * attn_decode_combine: one workgroup per (b, h, 32 head dims) merges the
//    splits of that head: M = max m_s, L = sum l_s 2^(m_s - M),
//    O = sum O_s 2^(m_s - M) / L, and writes the bf16 output and
//    lse = ln2 (M + log2 L).
// Cache lengths come from a device array (or are all S_max); a length above
// S_max counts as S_max, and an empty cache gives out = 0, lse = -inf.
// fp32 inputs take a plain one-thread-per-(b, h) kernel (exactness checks).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace sqa {
namespace {

using namespace dev;

constexpr int kBlk = 32;          // keys per block (one S^T MFMA tile)
constexpr int kWavesDec = 4;      // waves per workgroup (independent)
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
  int64_t n_waves;          // B * H_kv * HB * n_splits
  int S_max;
  int H_q;
  int H_kv;
  int R;
  int HB;                   // ceil(R / 32) query-head blocks per group
  int n_splits;
  int split_len;            // keys per split, multiple of kBlk
  float c;                  // |scale| * log2(e), > 0
  uint32_t q_sign;          // 0x8000 when scale < 0 (q negated on load, exact)
};

__device__ __forceinline__ int cache_len(const DecodeParams& p, int b) {
  const int len = p.seqlens ? p.seqlens[b] : p.S_max;
  return min(len, p.S_max);
}

template <int D>
__global__ __launch_bounds__(kWavesDec * 64, 2) void attn_decode_split_bf16(DecodeParams p) {
  constexpr int KS = D / 16;   // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;   // 32-dim blocks of O^T
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v[kWavesDec][2][kBlk * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // wave -> (b, split, head block, K/V head), K/V head fastest: waves that
  // run together read all heads of the same cache positions (whole rows)
  const int64_t wid = (int64_t)blockIdx.x * kWavesDec + wave;
  if (wid >= p.n_waves) return;   // wave-uniform; no barrier in this kernel
  const int g = (int)(wid % p.H_kv);
  const int64_t r1 = wid / p.H_kv;
  const int hb = (int)(r1 % p.HB);
  const int64_t r2 = r1 / p.HB;
  const int split = (int)(r2 % p.n_splits);
  const int b = (int)(r2 / p.n_splits);

  const int len = cache_len(p, b);
  const int k0 = split * p.split_len;
  if (k0 >= len) return;          // empty split: the combine step skips it
  const int k1 = min(k0 + p.split_len, len);
  const int n_blk = (k1 - k0 + kBlk - 1) / kBlk;

  const int hc = hb * 32 + col;   // query head of this lane's column, within the group
  const bool valid = hc < p.R;
  const int h = g * p.R + hc;

  const int64_t kv_stride = (int64_t)p.H_kv * D;
  const uint16_t* k_base = p.k + ((int64_t)b * p.S_max * p.H_kv + g) * D;
  const uint16_t* v_base = p.v + ((int64_t)b * p.S_max * p.H_kv + g) * D;

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

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
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
template <int D>
__global__ __launch_bounds__(256) void attn_decode_combine_bf16(DecodeParams p) {
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
  uint16_t* op = p.out + row * D + dc * 32;
  if (len <= 0) {   // uniform over the workgroup
    if (tid < 32) op[tid] = 0;
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
    bf16x4 w4;
#pragma unroll
    for (int e = 0; e < 4; ++e) w4[e] = (__bf16)(o[e] * inv);
    *(bf16x4*)(op + tid * 4) = w4;
    if (p.lse && dc == 0 && tid == 0) p.lse[row] = (M + log2f(Lt)) * 0.69314718055994531f;
  }
}

// fp32 path: one thread per (b, h), online softmax over the cache in fp32.
// Plain VALU arithmetic for exactness checks at small sizes.
template <int D>
__global__ __launch_bounds__(256) void attn_decode_f32(const float* __restrict__ q, const float* __restrict__ k,
                                                       const float* __restrict__ v, const int32_t* __restrict__ seqlens,
                                                       float* __restrict__ out, float* __restrict__ lse, int64_t B,
                                                       int S_max, int H_q, int H_kv, int R, float c) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= B * H_q) return;
  const int64_t b = t / H_q;
  const int h = (int)(t % H_q);
  const int g = h / R;
  int len = seqlens ? seqlens[b] : S_max;
  len = min(len, S_max);
  float* op = out + t * D;
  if (len <= 0) {
#pragma unroll
    for (int e = 0; e < D; ++e) op[e] = 0.f;
    if (lse) lse[t] = -__builtin_inff();
    return;
  }
  float qv[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = q[t * D + e];
    acc[e] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;
  for (int j = 0; j < len; ++j) {
    const float* kp = k + ((b * S_max + j) * H_kv + g) * D;
    const float* vp = v + ((b * S_max + j) * H_kv + g) * D;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) dot = __builtin_fmaf(qv[e], kp[e], dot);
    const float x = dot * c;
    const float m_new = fmaxf(m, x);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    const float pj = __builtin_amdgcn_exp2f(x - m_new);
    m = m_new;
    l = l * alpha + pj;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] = __builtin_fmaf(pj, vp[e], acc[e] * alpha);
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < D; ++e) op[e] = acc[e] * inv;
  if (lse) lse[t] = (m + log2f(l)) * 0.69314718055994531f;
}

template <int D>
hipError_t launch_decode_f32_t(const DecodeArgs& a) {
  const int64_t threads = a.B * a.H_q;
  // the fp32 kernel keeps the sign of the scale in c (no bf16 operand to negate)
  const float c = a.negate_q ? -a.c : a.c;
  hipLaunchKernelGGL((attn_decode_f32<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     (hipStream_t)a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v, a.seqlens,
                     (float*)a.out, a.lse, a.B, (int)a.S_max, a.H_q, a.H_kv, a.H_q / a.H_kv, c);
  return hipGetLastError();
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
  p.n_waves = a.B * a.H_kv * plan.head_blocks * plan.n_splits;
  p.c = a.c;
  p.q_sign = a.negate_q ? 0x8000u : 0u;
  const int64_t wgs = (p.n_waves + kWavesDec - 1) / kWavesDec;
  hipLaunchKernelGGL((attn_decode_split_bf16<D>), dim3((unsigned)wgs), dim3(kWavesDec * 64), 0,
                     (hipStream_t)a.stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = a.B * a.H_q;
  hipLaunchKernelGGL((attn_decode_combine_bf16<D>), dim3((unsigned)(rows * (D / 32))), dim3(256), 0,
                     (hipStream_t)a.stream, p);
  return hipGetLastError();
}

}  // namespace

// Split plan: about 8 waves per wave slot of the chip (8 per CU), so that
// the last round is a small part of the work even when many splits are
// empty (short caches).  Splits shorter than 512 keys are lengthened
// towards 512 as long as at least 2 waves per slot remain: short splits
// spend a larger share of their time starting up and add merge work (512
// instead of 256 made the 32/8 and 16/8 head configurations of a 4 x 128K
// cache 1-3 % faster).  Each split has at least 64 keys, and at least 16
// keys per query head it serves, so the fp32 partial results written per
// split stay within a few percent of the cache bytes it reads.
DecodePlan decode_plan(int64_t B, int64_t S_max, int32_t H_q, int32_t H_kv, int32_t d) {
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
  if (len < 64) len = 64;
  if (len < 16 * heads_per_wave) len = 16 * heads_per_wave;
  len = (len + kBlk - 1) / kBlk * kBlk;
  pl.split_len = (int)len;
  pl.n_splits = (int)(S_max > 0 ? (S_max + len - 1) / len : 1);
  pl.part_o_bytes = B * H_q * (int64_t)pl.n_splits * d * 4;
  pl.workspace_bytes = pl.part_o_bytes + B * H_q * (int64_t)pl.n_splits * 2 * 4;
  pl.n_waves = units * pl.n_splits;
  return pl;
}

hipError_t launch_attn_decode(const DecodeArgs& a) {
  if (a.dtype == 1) {
    switch (a.d) {
      case 32: return launch_decode_f32_t<32>(a);
      case 64: return launch_decode_f32_t<64>(a);
      case 128: return launch_decode_f32_t<128>(a);
    }
    return hipErrorInvalidValue;
  }
  const DecodePlan plan = decode_plan(a.B, a.S_max, a.H_q, a.H_kv, a.d);
  switch (a.d) {
    case 32: return launch_decode_t<32>(a, plan);
    case 64: return launch_decode_t<64>(a, plan);
    case 128: return launch_decode_t<128>(a, plan);
  }
  return hipErrorInvalidValue;
}

}  // namespace sqa
