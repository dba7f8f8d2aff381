// Decoupled-head attention backward for gfx950 (MI355X, CDNA4).
//
// Gradients of out = softmax(scale * Q K^T) V (per query head h, with K/V head
// g = floor(h / R) shared by the R query heads of its group, as in the GQA
// explainer's grouping figure and expand) for an upstream gradient dO:
//
//   P = exp(scale * S - lse),  dP = dO V^T,  D_i = <dO_i, O_i>,
//   dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO,
//
// where lse is the row log-normaliser the forward returns and dK, dV sum over
// the query heads of a group.  Three kernels:
//
//  * bwd_stats: D_i = <dO_i, O_i> and lse_i * log2(e), written per (b, head)
//    as contiguous, 64-padded rows of a caller-provided workspace, negated and
//    (lse) divided by c, so that the dK/dV kernel can start its score and dP
//    accumulators at them.
//  * bwd_dq: one wave per 32 query rows of one head; K/V tiles of 64 keys
//    staged in LDS for the whole K/V group (as in the forward).  With keys
//    along MFMA M (S^T = K Q^T, dP^T = V dO^T) each lane owns one query, so
//    D_i and lse_i are per-lane scalars; dQ^T += K^T dS^T reads K^T with
//    transposing LDS reads.
//  * bwd_dkdv: two waves per 32 keys of one K/V head, one per 32-query half
//    of each 64-row query tile (Q, dO and their statistics, for all R query
//    heads of the group, streamed through LDS); the workgroup's K and V rows
//    are staged once in LDS.  Each wave holds half the score state, so two
//    waves share a SIMD, and the halves' partial sums are added in LDS at
//    the end.  S = Q K^T and dP = dO V^T put keys on lanes, so
//    dV^T += dO^T P and dK^T += Q^T dS take P and dS straight from the
//    accumulators and dO^T, Q^T from transposing LDS reads.  The
//    accumulators start at -lse_i*log2(e)/c and -D_i, so they end at
//    s - lse2/c and dP - D: P = 2^(c acc) and dS = P acc' with no per-score
//    subtraction.
//
// bf16 inputs: all matrix products are bf16 MFMA with fp32 accumulation; P
// and dS are rounded to bf16 for the products that consume them.  fp32
// inputs: the same two-kernel split (bwd_dq_f32, bwd_dkdv_f32) on
// v_mfma_f32_32x32x2_f32, with P and dS kept in fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace sqa {
namespace {

using namespace dev;

constexpr int kRows32 = kBwdRows;  // query rows (dq) or keys (dk/dv) per wave
constexpr int kTile = 64;    // K/V tile (dq) and Q/dO tile (dk/dv) length
constexpr int kWaves = kBwdWaves;


struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  float* ws_lse2;    // [B, H_q, S_pad]: -lse * log2(e) / c  (pad rows -inf)
  float* ws_delta;   // [B, H_q, S_pad]: -<dO_i, O_i>        (pad rows 0)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int S;
  int S_pad;
  int H_q;
  int H_kv;
  int R;
  int n_groups;      // B * H_kv
  int n_items;       // dq: R * ceil(S / 32) per group
  int chunks;        // dq: workgroups per group
  int key_blocks;    // dk/dv: key blocks (workgroups) per group
  int kb_chunk;      // dk/dv: 0, or key blocks of one group that one XCD takes in a row
  float c;           // |scale| * log2(e)
  float scale;       // signed scale
  uint32_t q_sign;   // 0x8000 when scale < 0: q (dq kernel) or k (dk/dv kernel) negated on load, exact
};

// ---------------------------------------------------------------------------
// stats: delta and lse2 rows, transposed to [B, H_q, S_pad]; pad entries:
// delta 0, lse2 +inf.
// 8 lanes per (b, i, h) row.
template <int D>
__global__ __launch_bounds__(256) void bwd_stats_bf16(BwdParams p, int64_t B) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 3;  // over B * S_pad * H_q, ordered (b, h, i)
  const int sub = (int)(gid & 7);
  const int64_t total = B * p.H_q * (int64_t)p.S_pad;
  float acc = 0.f;
  int64_t b = 0, h = 0, i = 0;
  if (row < total) {
    i = row % p.S_pad;
    h = (row / p.S_pad) % p.H_q;
    b = row / ((int64_t)p.S_pad * p.H_q);
    if (i < p.S) {
      const int64_t off = ((b * p.S + i) * p.H_q + h) * D;
      for (int cc = sub; cc < D / 8; cc += 8) {
        const u32x4 ov = *(const u32x4*)(p.o + off + cc * 8);
        const u32x4 gv = *(const u32x4*)(p.dout + off + cc * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc += __uint_as_float(ov[e] << 16) * __uint_as_float(gv[e] << 16);
          acc += __uint_as_float(ov[e] & 0xFFFF0000u) * __uint_as_float(gv[e] & 0xFFFF0000u);
        }
      }
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < total && sub == 0) {
    const bool valid = i < p.S;
    // stored negated and (for lse) divided by c: they are the initial values
    // of the dK/dV kernel's score and dP accumulators, which then hold
    // s - lse2/c and dP - D directly.  Pad rows get -inf, so their
    // probabilities 2^(c (s - lse2/c)) are exactly 0 wherever they are
    // recomputed (no per-element tail mask).
    p.ws_delta[row] = valid ? -acc : 0.f;
    p.ws_lse2[row] = valid ? -(p.lse[(b * p.S + i) * p.H_q + h] * 1.4426950408889634f) / p.c : -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------
// dQ: 4 waves per workgroup, one 32-row item each (as in the forward).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16(BwdParams p) {
  constexpr int WAVES = kWaves, KEYS = kTile;
  constexpr int KS = D / 16, DB = D / 32, NB = KEYS / 32, NT = KEYS / 16;
  constexpr int TILE = KEYS * D;
  // the four K/V tile buffers in one LDS block, so that each read is one
  // per-lane offset plus an immediate (separate arrays cost an address
  // register per buffer and spilled at d = 128)
  __shared__ __attribute__((aligned(1024))) uint16_t lds_all[4 * TILE];
  uint16_t* const lds_k0 = lds_all;
  uint16_t* const lds_k1 = lds_all + TILE;
  uint16_t* const lds_v0 = lds_all + 2 * TILE;
  uint16_t* const lds_v1 = lds_all + 3 * TILE;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  const int S = p.S;

  const int grp = blockIdx.x % p.n_groups;
  const int ord = blockIdx.x / p.n_groups;
  const int chunk = CAUSAL ? (p.chunks - 1 - ord) : ord;
  const int b = grp / p.H_kv;
  const int g = grp % p.H_kv;
  const int item = chunk * WAVES + wave;
  const bool active = item < p.n_items;
  const int pos0 = (item / p.R) * kRows32;
  const int h = active ? g * p.R + item % p.R : 0;
  const int last_item = min(chunk * WAVES + WAVES - 1, p.n_items - 1);
  const int wg_last_pos = min((last_item / p.R) * kRows32 + kRows32 - 1, S - 1);
  const int n_tiles = CAUSAL ? wg_last_pos / KEYS + 1 : (S + KEYS - 1) / KEYS;

  const int64_t kv_stride = (int64_t)p.H_kv * D;
  const uint16_t* k_base = p.k + ((int64_t)b * S * p.H_kv + g) * D;
  const uint16_t* v_base = p.v + ((int64_t)b * S * p.H_kv + g) * D;
  TileCopy<D, WAVES, KEYS> cp;
  cp.init(kv_stride, wave, lane);
  cp.issue(k_base, kv_stride, S, (SQA_LDS uint16_t*)lds_k0, wave);
  cp.issue(v_base, kv_stride, S, (SQA_LDS uint16_t*)lds_v0, wave);

  // Q^T and dO^T as B operands: lane holds query pos0 + col, dims ks*16 + half*8 ...
  const int qrow = min(pos0 + col, S - 1);
  bf16x8 qf[KS], gf[KS];
  {
    const int64_t off = (((int64_t)b * S + qrow) * p.H_q + h) * D + half * 8;
    const uint32_t sgn = p.q_sign * 0x10001u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = *(const u32x4*)(p.q + off + ks * 16);
      raw ^= (u32x4){sgn, sgn, sgn, sgn};
      qf[ks] = __builtin_bit_cast(bf16x8, raw);
      gf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(p.dout + off + ks * 16));
    }
  }
  const int64_t srow = ((int64_t)b * p.H_q + h) * p.S_pad + qrow;
  const float lse2 = -p.c * p.ws_lse2[srow];   // the workspace holds -lse2/c and -D
  const float delta = -p.ws_delta[srow];

  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = tile_off<D>(col, ks * 16 + half * 8);
  int t_off[DB][2];
  {
    const int grp16 = lane >> 4, i16 = lane & 15, e = i16 >> 2, c4 = i16 & 3;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 2; ++j) t_off[db][j] = tile_off<D>(4 * half + 8 * j + e, db * 32 + (grp16 & 1) * 16 + 4 * c4);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = (f32x16){};
  const float c = p.c;
  const int my_q = pos0 + col;
  const int wave_last = pos0 + kRows32 - 1;

  auto step = [&](int t, SQA_LDS uint16_t* kt, SQA_LDS uint16_t* vt, SQA_LDS uint16_t* kn, SQA_LDS uint16_t* vn) {
    const int kv0 = t * KEYS;
    wait_copies();
    __syncthreads();
    if (t + 1 < n_tiles) {
      const int64_t nxt = (int64_t)(kv0 + KEYS) * kv_stride;
      cp.issue(k_base + nxt, kv_stride, S - kv0 - KEYS, kn, wave);
      cp.issue(v_base + nxt, kv_stride, S - kv0 - KEYS, vn, wave);
    }
    if (!active || (CAUSAL && kv0 > wave_last)) return;
    // S^T = K Q^T and dP^T = V dO^T (keys along M, this lane's query along N)
    f32x16 s[NB], dp[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb] = dp[nb] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 a = *(const SQA_LDS bf16x8*)(kt + nb * 32 * D + k_off[ks]);
        s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[nb], 0, 0, 0);
        const bf16x8 bv = *(const SQA_LDS bf16x8*)(vt + nb * 32 * D + k_off[ks]);
        dp[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, gf[ks], dp[nb], 0, 0, 0);
      }
    lds_mfma_pipeline_hint<2 * KS * NB, 1, 4>();
    // P = 2^(c s - lse2), masked keys 0; dS = P (dP - D); key of s[nb][r] is
    // kv0 + 4*half + nb*32 + 8*(r/4) + r%4
    // masked scores go to -inf (P = 0) in a pass of their own, taken only on
    // tiles that hold a masked key
    const bool need_mask = (kv0 + KEYS > S) || (CAUSAL && kv0 + KEYS - 1 > pos0);
    if (__builtin_expect(need_mask, 0)) {
      asm volatile("" ::: "memory");  // keeps this pass a branch (no if-conversion into selects)
      const int lim = (CAUSAL ? min(my_q, S - 1) : S - 1) - kv0 - 4 * half;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (nb * 32 + 8 * (r >> 2) + (r & 3) > lim) s[nb][r] = -__builtin_inff();
    }
    // exponentials through the dQ MFMAs ahead of the SIMD's other wave
    // (as in the forward): 2 % faster at d = 128, same results
    __builtin_amdgcn_s_setprio(2);
    bf16x8 dsk[NT];
#pragma unroll
    for (int st = 0; st < NT; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int nb = st >> 1, r = (st & 1) * 8 + e;
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][r], c, -lse2));
        dsk[st][e] = (__bf16)(pv * (dp[nb][r] - delta));
      }
    // dQ^T += K^T dS^T (K^T from transposing reads of the K tile)
#pragma unroll
    for (int st = 0; st < NT; ++st)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SQA_LDS bf16x4*)(kt + st * 16 * D + t_off[db][0]));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SQA_LDS bf16x4*)(kt + st * 16 * D + t_off[db][1]));
        const bf16x8 ka = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, dsk[st], acc[db], 0, 0, 0);
      }
    lds_mfma_pipeline_hint<NT * DB, 2, 4>();
    __builtin_amdgcn_s_setprio(0);
  };
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, (SQA_LDS uint16_t*)lds_k0, (SQA_LDS uint16_t*)lds_v0, (SQA_LDS uint16_t*)lds_k1, (SQA_LDS uint16_t*)lds_v1);
    if (t + 1 < n_tiles)
      step(t + 1, (SQA_LDS uint16_t*)lds_k1, (SQA_LDS uint16_t*)lds_v1, (SQA_LDS uint16_t*)lds_k0, (SQA_LDS uint16_t*)lds_v0);
  }

  if (!active || my_q >= S) return;
  uint16_t* op = p.dq + (((int64_t)b * S + my_q) * p.H_q + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][4 * j + e] * p.scale);
      *(bf16x4*)(op + db * 32 + 8 * j + 4 * half) = w;
    }
}

// ---------------------------------------------------------------------------
// dK, dV: 8 waves per workgroup and 128 keys.  Wave w takes keys (w % 4) * 32
// ... +31 and query half w / 4 of every 64-row query tile, so each wave holds
// the score and dP accumulators of 32 queries only and two waves share each
// SIMD: the other wave's matrix products fill the gaps of this one's
// softmax.  The two halves' partial dK, dV are added through LDS at the end,
// in a fixed order.
// Copies of one query tile: Q rows and dO rows of head h (TileCopy), plus
// the 256-byte runs of lse2 and delta, one copy each from its own 64-bit base
// (lanes 0-15 carry the run; the others repeat it into unused LDS).
template <int D, bool CAUSAL, int MIN_WAVES_PER_SIMD>
__global__ __launch_bounds__(512, MIN_WAVES_PER_SIMD) void bwd_dkdv_bf16(BwdParams p) {
  constexpr int WAVES = 2 * kWaves, QT = kTile;
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int TILE = QT * D;
  constexpr int KEYS_WG = kWaves * kRows32;
  // waves that copy the query tiles: all 8, or 4 when a tile is only 4
  // wave-wide copies (d = 32)
  constexpr int CW = (QT * D / 8 / 64) >= WAVES ? WAVES : kWaves;
  // one LDS block with the four Q / dO tile buffers first, so that every
  // read of them is one per-lane offset plus an immediate below 64 KiB (with
  // separate arrays the compiler kept an address per buffer and spilled)
  constexpr int TB = TILE * 2;          // bytes per tile buffer
  constexpr int KVB = KEYS_WG * D * 2;  // bytes of the workgroup's K (or V) rows
  __shared__ __attribute__((aligned(1024))) uint8_t lds_all[4 * TB + 2 * KVB + 2 * 2048];
  uint16_t* const lds_q0 = (uint16_t*)(lds_all + 0 * TB);
  uint16_t* const lds_q1 = (uint16_t*)(lds_all + 1 * TB);
  uint16_t* const lds_g0 = (uint16_t*)(lds_all + 2 * TB);
  uint16_t* const lds_g1 = (uint16_t*)(lds_all + 3 * TB);
  uint16_t* const lds_kk = (uint16_t*)(lds_all + 4 * TB);
  uint16_t* const lds_vv = (uint16_t*)(lds_all + 4 * TB + KVB);
  float* const lds_s0 = (float*)(lds_all + 4 * TB + 2 * KVB);          // [0,64) lse2, [256,320) delta
  float* const lds_s1 = (float*)(lds_all + 4 * TB + 2 * KVB + 2048);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = wave % kWaves;  // key block of this wave
  const int qh = wave / kWaves;  // query half of each tile
  const int half = lane >> 5;
  const int col = lane & 31;
  const int S = p.S;

  // workgroup -> (group, key block); low keys first, as they see the most
  // queries when causal.  With kb_chunk set, workgroups dealt to one XCD
  // (blockIdx mod 8 under round-robin dispatch) take kb_chunk consecutive
  // key blocks of one group, so that the query tiles in flight on that XCD
  // span 2 * kb_chunk tiles of a head and stay in its L2.  Chunks go to XCDs
  // heaviest first, the order reversed every other round to balance the
  // XCDs; workgroups past the last key block exit at once.
  int grp, kb;
  if (p.kb_chunk) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int round = slot / p.kb_chunk;
    const int unit = round * 8 + ((round & 1) ? 7 - xcd : xcd);
    grp = unit % p.n_groups;
    kb = (unit / p.n_groups) * p.kb_chunk + slot % p.kb_chunk;
    if (kb >= p.key_blocks) return;
  } else {
    grp = blockIdx.x % p.n_groups;
    kb = blockIdx.x / p.n_groups;
  }
  const int b = grp / p.H_kv;
  const int g = grp % p.H_kv;
  const int key_wg0 = kb * KEYS_WG;
  const int key0 = key_wg0 + kw * kRows32;
  const int my_key = key0 + col;

  // query tiles: R heads x tiles from the first one that can see this block
  const int qt_first = CAUSAL ? key_wg0 / QT : 0;
  const int qt_count = (S + QT - 1) / QT - qt_first;
  const int U = p.R * qt_count;

  const int64_t q_stride = (int64_t)p.H_q * D;
  TileCopy<D, CW, QT> cp;
  if (wave < CW) cp.init(q_stride, wave, lane);
  // statistics of a tile: two 256-byte runs (lse2, delta) at 64-bit bases;
  // lanes 16-63 repeat lanes 0-15 into the unused rest of each 1 KiB half
  const uint32_t stat_lane = (uint32_t)(lane & 15) * 16u;

  auto issue_tile = [&](int u, SQA_LDS uint16_t* qd, SQA_LDS uint16_t* gd, SQA_LDS float* sd) {
    const int hl = u / qt_count;
    const int qt = qt_first + u % qt_count;
    const int h = g * p.R + hl;
    const int64_t base = (((int64_t)b * S + qt * QT) * p.H_q + h) * D;
    if (wave < CW) {
      cp.issue(p.q + base, q_stride, S - qt * QT, qd, wave);
      cp.issue(p.dout + base, q_stride, S - qt * QT, gd, wave);
    }
    if (wave == 0) {
      const int64_t srow = ((int64_t)b * p.H_q + h) * p.S_pad + qt * QT;
      dma16(p.ws_lse2 + srow, stat_lane, lds_addr(sd));
      dma16(p.ws_delta + srow, stat_lane, lds_addr(sd + 256));
    }
  };

  // K and V rows of the workgroup's keys go to LDS once (K's sign flipped
  // for a negative scale, so that c * s = scale * log2(e) * <q, k> with
  // c = |scale| * log2(e)); the half-0 waves write them, both halves read
  // them as B operands (lane holds key my_key, dims ks*16 + half*8 ...)
  // after the first tile's barrier.
  if (qh == 0) {
    const int krow = min(my_key, S - 1);
    const int64_t off = (((int64_t)b * S + krow) * p.H_kv + g) * D + half * 8;
    const uint32_t sgn = p.q_sign * 0x10001u;
    const int row = kw * kRows32 + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = *(const u32x4*)(p.k + off + ks * 16);
      raw ^= (u32x4){sgn, sgn, sgn, sgn};
      *(SQA_LDS u32x4*)((SQA_LDS uint16_t*)lds_kk + tile_off<D>(row, ks * 16 + half * 8)) = raw;
      *(SQA_LDS u32x4*)((SQA_LDS uint16_t*)lds_vv + tile_off<D>(row, ks * 16 + half * 8)) =
          *(const u32x4*)(p.v + off + ks * 16);
    }
  }
  if (U > 0) issue_tile(0, (SQA_LDS uint16_t*)lds_q0, (SQA_LDS uint16_t*)lds_g0, (SQA_LDS float*)lds_s0);

  // row col of a 32-row block (a Q / dO half, or this wave's K / V rows):
  // the swizzle depends on the low 4 row bits only, so one offset per k-step
  // serves every block; the blocks' bases are wave-uniform
  int c_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) c_off[ks] = tile_off<D>(col, ks * 16 + half * 8);
  const SQA_LDS uint16_t* kk_w = (const SQA_LDS uint16_t*)lds_kk + kw * kRows32 * D;
  const SQA_LDS uint16_t* vv_w = (const SQA_LDS uint16_t*)lds_vv + kw * kRows32 * D;
  const int qh_base = qh * 32 * D;
  // transposing reads of the Q / dO half: offsets of head-dim block 0; block
  // db is the same offset with bit 5 replaced by db's bits (the swizzle
  // leaves chunk bits 2-3 of these columns to db)
  int t_off0[2];
  {
    const int grp16 = lane >> 4, i16 = lane & 15, e = i16 >> 2, c4 = i16 & 3;
#pragma unroll
    for (int j = 0; j < 2; ++j) t_off0[j] = tile_off<D>(4 * half + 8 * j + e, (grp16 & 1) * 16 + 4 * c4);
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = (f32x16){};
  const float c = p.c;

  auto step = [&](int u, SQA_LDS uint16_t* qt_l, SQA_LDS uint16_t* gt_l, SQA_LDS float* st_l, SQA_LDS uint16_t* qn,
                  SQA_LDS uint16_t* gn, SQA_LDS float* sn) {
    wait_copies();
    __syncthreads();
    if (u + 1 < U) issue_tile(u + 1, qn, gn, sn);
    const int qt = qt_first + u % qt_count;
    const int qbase = qt * QT + qh * 32;
    // this half before the wave's keys (causal) or past the end
    if (CAUSAL ? qbase + 31 < key0 : qbase >= S) return;
    // S - lse2/c = Q K^T + (-lse2/c) and dP - D = dO V^T + (-D): the row
    // statistics (stored negated, lse2 divided by c) start the accumulators
    // (queries along M, this lane's key along N)
    f32x16 s, dp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 a = *(const SQA_LDS f32x4*)(st_l + qh * 32 + 8 * j + 4 * half);
      const f32x4 d4 = *(const SQA_LDS f32x4*)(st_l + 256 + qh * 32 + 8 * j + 4 * half);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[4 * j + e] = a[e];
        dp[4 * j + e] = d4[e];
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *(const SQA_LDS bf16x8*)(qt_l + qh_base + c_off[ks]);
      const bf16x8 kb8 = *(const SQA_LDS bf16x8*)(kk_w + c_off[ks]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kb8, s, 0, 0, 0);
      const bf16x8 ga = *(const SQA_LDS bf16x8*)(gt_l + qh_base + c_off[ks]);
      const bf16x8 vb = *(const SQA_LDS bf16x8*)(vv_w + c_off[ks]);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vb, dp, 0, 0, 0);
    }
    // the accumulators of rows past S start at -inf (P = 0); only the
    // causal mask is explicit, in a pass of its own (a branch, not selects)
    const bool need_mask = CAUSAL && qbase < key0 + 31;
    if (__builtin_expect(need_mask, 0)) {
      asm volatile("" ::: "memory");
      const int qlo = qbase + 4 * half;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (my_key > qlo + 8 * (r >> 2) + (r & 3)) s[r] = -__builtin_inff();
    }
    // P and dS = P (dP - D), rounded to bf16; query of register r:
    // qbase + 8*(r/4) + 4*half + r%4
    // the 4-waves-per-SIMD build issues its exponentials and dV/dK MFMAs
    // ahead of the SIMD's other waves (7-11 % faster there; no gain, or a
    // loss, at 2 waves per SIMD)
    if constexpr (MIN_WAVES_PER_SIMD == 4) __builtin_amdgcn_s_setprio(2);
    bf16x8 pk[2], dsk[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = st * 8 + e;
        const float pv = __builtin_amdgcn_exp2f(s[r] * c);
        pk[st][e] = (__bf16)pv;
        dsk[st][e] = (__bf16)(pv * dp[r]);
      }
    // dV^T += dO^T P and dK^T += Q^T dS (16 queries per MFMA step)
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int ro = qh_base + st * 16 * D;
        const int t0 = t_off0[0] ^ (db << 5), t1 = t_off0[1] ^ (db << 5);
        const bf16x4 glo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SQA_LDS bf16x4*)(gt_l + ro + t0));
        const bf16x4 ghi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SQA_LDS bf16x4*)(gt_l + ro + t1));
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(glo, ghi, 0, 1, 2, 3, 4, 5, 6, 7),
                                                         pk[st], dv[db], 0, 0, 0);
        const bf16x4 qlo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SQA_LDS bf16x4*)(qt_l + ro + t0));
        const bf16x4 qhi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SQA_LDS bf16x4*)(qt_l + ro + t1));
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(qlo4, qhi4, 0, 1, 2, 3, 4, 5, 6, 7),
                                                         dsk[st], dk[db], 0, 0, 0);
      }
    if constexpr (MIN_WAVES_PER_SIMD == 4) __builtin_amdgcn_s_setprio(0);
  };
  for (int u = 0; u < U; u += 2) {
    step(u, (SQA_LDS uint16_t*)lds_q0, (SQA_LDS uint16_t*)lds_g0, (SQA_LDS float*)lds_s0, (SQA_LDS uint16_t*)lds_q1,
         (SQA_LDS uint16_t*)lds_g1, (SQA_LDS float*)lds_s1);
    if (u + 1 < U)
      step(u + 1, (SQA_LDS uint16_t*)lds_q1, (SQA_LDS uint16_t*)lds_g1, (SQA_LDS float*)lds_s1,
           (SQA_LDS uint16_t*)lds_q0, (SQA_LDS uint16_t*)lds_g0, (SQA_LDS float*)lds_s0);
  }

  // the half-1 waves hand their partial sums to the half-0 waves of the same
  // keys through LDS (all tiles consumed, so the buffers are free): 16 KiB
  // (d = 128) per array and wave, lane-contiguous 16-byte chunks
  __syncthreads();
  constexpr int RB = 64 * DB * 16;  // floats per wave and array
  static_assert(RB * 4 <= TB && 2 * RB * 4 <= KVB, "reduction slots exceed the LDS buffers");
  SQA_LDS float* red_k;
  SQA_LDS float* red_v;
  if (kw == 0) {
    red_k = (SQA_LDS float*)lds_q0;
    red_v = (SQA_LDS float*)lds_q1;
  } else if (kw == 1) {
    red_k = (SQA_LDS float*)lds_g0;
    red_v = (SQA_LDS float*)lds_g1;
  } else if (kw == 2) {
    red_k = (SQA_LDS float*)lds_kk;
    red_v = (SQA_LDS float*)lds_kk + RB;
  } else {
    red_k = (SQA_LDS float*)lds_vv;
    red_v = (SQA_LDS float*)lds_vv + RB;
  }
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *(SQA_LDS f32x4*)(red_k + ((db * 4 + j) * 64 + lane) * 4) =
            (f32x4){dk[db][4 * j], dk[db][4 * j + 1], dk[db][4 * j + 2], dk[db][4 * j + 3]};
        *(SQA_LDS f32x4*)(red_v + ((db * 4 + j) * 64 + lane) * 4) =
            (f32x4){dv[db][4 * j], dv[db][4 * j + 1], dv[db][4 * j + 2], dv[db][4 * j + 3]};
      }
  }
  __syncthreads();
  if (qh == 1 || my_key >= S) return;
  const int64_t off = (((int64_t)b * S + my_key) * p.H_kv + g) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 ok = *(const SQA_LDS f32x4*)(red_k + ((db * 4 + j) * 64 + lane) * 4);
      const f32x4 ov = *(const SQA_LDS f32x4*)(red_v + ((db * 4 + j) * 64 + lane) * 4);
      bf16x4 wk, wv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wk[e] = (__bf16)((dk[db][4 * j + e] + ok[e]) * p.scale);
        wv[e] = (__bf16)(dv[db][4 * j + e] + ov[e]);
      }
      *(bf16x4*)(p.dk + off + db * 32 + 8 * j + 4 * half) = wk;
      *(bf16x4*)(p.dv + off + db * 32 + 8 * j + 4 * half) = wv;
    }
}

// ---------------------------------------------------------------------------
// fp32 path: row statistics as above (plain fp32 loop), then dq and dk/dv on
// the fp32 matrix cores.
template <int D>
__global__ __launch_bounds__(256) void bwd_stats_f32(const float* o, const float* dout, const float* lse, float* ws_lse2,
                                                     float* ws_delta, int64_t B, int S, int S_pad, int H_q) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b, h, i) over S_pad
  if (row >= B * H_q * (int64_t)S_pad) return;
  const int64_t i = row % S_pad, h = (row / S_pad) % H_q, b = row / ((int64_t)S_pad * H_q);
  if (i >= S) {
    ws_lse2[row] = 0.f;
    ws_delta[row] = 0.f;
    return;
  }
  const int64_t off = ((b * S + i) * H_q + h) * D;
  float acc = 0.f;
  for (int e = 0; e < D; ++e) acc = __builtin_fmaf(o[off + e], dout[off + e], acc);
  ws_delta[row] = acc;
  ws_lse2[row] = lse[(b * S + i) * H_q + h] * 1.4426950408889634f;
}

struct F32BwdParams {
  const float* q;
  const float* k;
  const float* v;
  const float* dout;
  const float* ws_lse2;   // [B, H_q, S_pad] lse * log2(e)
  const float* ws_delta;  // [B, H_q, S_pad] D_i = <dO_i, O_i>
  float* dq;
  float* dk;
  float* dv;
  int S;
  int S_pad;
  int H_q;
  int H_kv;
  int R;
  int n_groups;   // B * H_kv
  int n_items;    // R * ceil(S / 32), query items per group (dq)
  int chunks;     // ceil(n_items / 4), dq workgroups per group
  int key_blocks; // ceil(S / 128), dk/dv workgroups per group
  float c;        // |scale| * log2(e), strictly positive (a tiny value when scale == 0)
  uint32_t neg;   // 0x80000000 when scale < 0: the S product's register operand is negated
  float scale;
};

// dq on v_mfma_f32_32x32x2_f32, in the forward fp32 kernel's layout: a
// workgroup of 4 waves owns one K/V group and 4 items of 32 query rows; K
// and V tiles of 32 keys pass through LDS.  Per tile and wave,
// S^T = K Q^T and dP^T = V dO^T (keys along M, this lane's query along N, so
// lse and D_i are per-lane scalars), P = 2^(c s - lse2), dS = P (dP - D_i),
// and dQ^T += K^T dS^T with the dS register r as the B operand for the key
// pair 8*(r/4) + r%4 and + 4 (the two wave halves).  dq = scale * dQ.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_f32(F32BwdParams p) {
  constexpr int WAVES = 4, KP = D / 2, DB = D / 32, KB = 32, LD = F32Tile<D>::LD;
  __shared__ float lds_k[2][KB * LD];
  __shared__ float lds_v[2][KB * LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  const int S = p.S;
  const int grp = blockIdx.x % p.n_groups;
  const int ord = blockIdx.x / p.n_groups;
  const int chunk = CAUSAL ? (p.chunks - 1 - ord) : ord;
  const int b = grp / p.H_kv;
  const int g = grp % p.H_kv;
  const int item = chunk * WAVES + wave;
  const bool active = item < p.n_items;
  const int pos0 = (item / p.R) * 32;
  const int h = g * p.R + item % p.R;
  const int last_item = min(chunk * WAVES + WAVES - 1, p.n_items - 1);
  const int wg_last_pos = min((last_item / p.R) * 32 + 31, S - 1);
  const int n_tiles = CAUSAL ? wg_last_pos / KB + 1 : (S + KB - 1) / KB;
  const int my_q = pos0 + col;

  const int64_t kv_stride = (int64_t)p.H_kv * D;
  const float* k_base = p.k + (int64_t)b * S * kv_stride + g * D;
  const float* v_base = p.v + (int64_t)b * S * kv_stride + g * D;
  F32Tile<D> tk, tv;
  tk.load(k_base, kv_stride, 0, S, tid);
  tv.load(v_base, kv_stride, 0, S, tid);

  // this lane's query row: Q^T (negated for a negative scale, so that the
  // masks' -inf scores stay -inf with c > 0) and dO^T operands (dims
  // 2*ks + half), lse2 (+inf for rows past S, so that their P is exactly 0)
  // and D_i
  float qf[KP], gf[KP];
  float lse2 = __builtin_inff(), delta = 0.f;
  {
    const int qrow = min(my_q, S - 1);
    const int64_t off = (((int64_t)b * S + qrow) * p.H_q + h) * D + half;
#pragma unroll
    for (int ks = 0; ks < KP; ++ks) {
      qf[ks] = __uint_as_float(__float_as_uint(p.q[off + 2 * ks]) ^ p.neg);
      gf[ks] = p.dout[off + 2 * ks];
    }
    if (active && my_q < S) {
      const int64_t srow = ((int64_t)b * p.H_q + h) * p.S_pad + my_q;
      lse2 = p.ws_lse2[srow];
      delta = p.ws_delta[srow];
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  const float c = p.c;
  const int wave_last = pos0 + 31;

  tk.store(lds_k[0], tid);
  tv.store(lds_v[0], tid);
  if (n_tiles > 1) {
    tk.load(k_base, kv_stride, KB, S, tid);
    tv.load(v_base, kv_stride, KB, S, tid);
  }
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    __syncthreads();   // tile t stored by everyone; tile t-1 fully consumed
    if (t + 1 < n_tiles) {
      tk.store(lds_k[buf ^ 1], tid);
      tv.store(lds_v[buf ^ 1], tid);
    }
    if (t + 2 < n_tiles) {
      tk.load(k_base, kv_stride, (t + 2) * KB, S, tid);
      tv.load(v_base, kv_stride, (t + 2) * KB, S, tid);
    }
    const int kv0 = t * KB;
    if (!active || (CAUSAL && kv0 > wave_last)) continue;
    const float* kt = lds_k[buf];
    const float* vt = lds_v[buf];
    f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KP; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kt[col * LD + 2 * ks + half], qf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vt[col * LD + 2 * ks + half], gf[ks], dp, 0, 0, 0);
    }
    // s[r] holds key kv0 + 8*(r/4) + 4*half + r%4
    if ((kv0 + KB > S) || (CAUSAL && kv0 + KB - 1 > pos0)) {
      const int lim = (CAUSAL ? min(my_q, S - 1) : S - 1) - kv0 - 4 * half;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) > lim) s[r] = -__builtin_inff();
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lse2)) * (dp[r] - delta);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * half + (r & 3);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(kt[key * LD + db * 32 + col], s[r], o[db], 0, 0, 0);
    }
  }

  if (!active || my_q >= S) return;
  float* op = p.dq + (((int64_t)b * S + my_q) * p.H_q + h) * D;
  const float sc = p.scale;
  // dQ^T[db] register r holds head dim db*32 + 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(f32x4*)(op + db * 32 + 8 * j + 4 * half) =
          (f32x4){o[db][4 * j] * sc, o[db][4 * j + 1] * sc, o[db][4 * j + 2] * sc, o[db][4 * j + 3] * sc};
}

// dk and dv on v_mfma_f32_32x32x2_f32: a workgroup of 4 waves owns 128 keys
// of one K/V group, each wave 32 of them with their K^T and V^T operands in
// registers (this lane's key, dims 2*ks + half).  Tiles of 32 query rows of
// Q and dO, with their lse2 and D_i, stream through LDS for all R query
// heads of the group, so the sum over the group happens in registers.  Per
// tile and wave, S = Q K^T and dP = dO V^T (queries along M, this lane's key
// along N), P = 2^(c s - lse2_i), dS = P (dP - D_i), then dV^T += dO^T P and
// dK^T += Q^T dS with the register r as the B operand for the query pair
// 8*(r/4) + r%4 and + 4.  dk = scale * dK.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_f32(F32BwdParams p) {
  constexpr int KP = D / 2, DB = D / 32, QT = 32, LD = F32Tile<D>::LD;
  __shared__ float lds_q[2][QT * LD];
  __shared__ float lds_g[2][QT * LD];
  __shared__ float lds_st[2][2 * QT];   // [lse2 x 32 | D_i x 32]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  const int S = p.S;
  const int grp = blockIdx.x % p.n_groups;
  const int kb = blockIdx.x / p.n_groups;
  const int b = grp / p.H_kv;
  const int g = grp % p.H_kv;
  const int key_wg0 = kb * 128;
  const int wave_key0 = key_wg0 + wave * 32;
  const int my_key = wave_key0 + col;

  const int qt_first = CAUSAL ? key_wg0 / QT : 0;
  const int qt_count = (S + QT - 1) / QT - qt_first;
  const int U = p.R * qt_count;

  const int64_t q_stride = (int64_t)p.H_q * D;
  F32Tile<D> tq, tg;
  float st_val = __builtin_inff();
  auto load = [&](int u) {
    const int h = g * p.R + u / qt_count;
    const int row0 = (qt_first + u % qt_count) * QT;
    const int64_t base = ((int64_t)b * S * p.H_q + h) * D;
    tq.load(p.q + base, q_stride, row0, S, tid);
    tg.load(p.dout + base, q_stride, row0, S, tid);
    if (tid < 2 * QT) {   // lse2 (+inf past S: P = 0) and D_i of the tile's rows
      const int i = row0 + (tid & (QT - 1));
      const int64_t srow = ((int64_t)b * p.H_q + h) * p.S_pad + min(i, S - 1);
      st_val = tid < QT ? (i < S ? p.ws_lse2[srow] : __builtin_inff()) : p.ws_delta[srow];
    }
  };
  auto store = [&](int buf) {
    tq.store(lds_q[buf], tid);
    tg.store(lds_g[buf], tid);
    if (tid < 2 * QT) lds_st[buf][tid] = st_val;
  };

  // this lane's key: K^T (negated for a negative scale: the S product only;
  // dK uses Q as given) and V^T operands (rows past S clamped; not stored)
  float kf[KP], vf[KP];
  {
    const int64_t off = (((int64_t)b * S + min(my_key, S - 1)) * p.H_kv + g) * D + half;
#pragma unroll
    for (int ks = 0; ks < KP; ++ks) {
      kf[ks] = __uint_as_float(__float_as_uint(p.k[off + 2 * ks]) ^ p.neg);
      vf[ks] = p.v[off + 2 * ks];
    }
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = (f32x16){};
  const float c = p.c;

  if (U > 0) {
    load(0);
    store(0);
  }
  if (U > 1) load(1);
  for (int u = 0; u < U; ++u) {
    const int buf = u & 1;
    __syncthreads();   // tile u stored by everyone; tile u-1 fully consumed
    if (u + 1 < U) store(buf ^ 1);
    if (u + 2 < U) load(u + 2);
    const int qbase = (qt_first + u % qt_count) * QT;
    // every query of the tile before this wave's keys (causal): no work
    if (CAUSAL && qbase + QT - 1 < wave_key0) continue;
    const float* qt = lds_q[buf];
    const float* gt = lds_g[buf];
    const float* st = lds_st[buf];
    f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KP; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(qt[col * LD + 2 * ks + half], kf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x2f32(gt[col * LD + 2 * ks + half], vf[ks], dp, 0, 0, 0);
    }
    // register r: query qbase + 8*(r/4) + 4*half + r%4
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = 8 * (r >> 2) + 4 * half + (r & 3);
      if (CAUSAL && my_key > qbase + qi) s[r] = -__builtin_inff();
      s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -st[qi]));
      ds[r] = s[r] * (dp[r] - st[QT + qi]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = 8 * (r >> 2) + 4 * half + (r & 3);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(gt[qi * LD + db * 32 + col], s[r], dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(qt[qi * LD + db * 32 + col], ds[r], dk[db], 0, 0, 0);
      }
    }
  }

  if (my_key >= S) return;
  const int64_t off = (((int64_t)b * S + my_key) * p.H_kv + g) * D;
  const float sc = p.scale;
  // dK^T / dV^T[db] register r holds head dim db*32 + 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = db * 32 + 8 * j + 4 * half;
      *(f32x4*)(p.dk + off + e) =
          (f32x4){dk[db][4 * j] * sc, dk[db][4 * j + 1] * sc, dk[db][4 * j + 2] * sc, dk[db][4 * j + 3] * sc};
      *(f32x4*)(p.dv + off + e) = (f32x4){dv[db][4 * j], dv[db][4 * j + 1], dv[db][4 * j + 2], dv[db][4 * j + 3]};
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_bf16_t(const BwdArgs& a) {
  BwdParams p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.o = (const uint16_t*)a.out;
  p.dout = (const uint16_t*)a.dout;
  p.lse = a.lse;
  p.S = (int)a.S;
  p.S_pad = (int)pad64(a.S);
  p.H_q = a.H_q;
  p.H_kv = a.H_kv;
  p.R = a.H_q / a.H_kv;
  p.ws_lse2 = (float*)a.workspace;
  p.ws_delta = (float*)a.workspace + a.B * a.H_q * (int64_t)p.S_pad;
  p.dq = (uint16_t*)a.dq;
  p.dk = (uint16_t*)a.dk;
  p.dv = (uint16_t*)a.dv;
  p.n_groups = (int)(a.B * a.H_kv);
  p.n_items = p.R * (int)((a.S + kRows32 - 1) / kRows32);
  p.chunks = (p.n_items + kWaves - 1) / kWaves;
  p.key_blocks = (int)((a.S + kWaves * kRows32 - 1) / (kWaves * kRows32));
  p.c = a.c;
  p.scale = a.scale;
  p.q_sign = a.negate_q ? 0x8000u : 0u;
  hipStream_t st = (hipStream_t)a.stream;
  const int64_t stat_threads = a.B * a.H_q * (int64_t)p.S_pad * 8;
  hipLaunchKernelGGL((bwd_stats_bf16<D>), dim3((unsigned)((stat_threads + 255) / 256)), dim3(256), 0, st, p, a.B);
  hipLaunchKernelGGL((bwd_dq_bf16<D, CAUSAL>), dim3((unsigned)((int64_t)p.n_groups * p.chunks)), dim3(kWaves * 64), 0,
                     st, p);
  const int64_t dkdv_grid = dkdv_layout(p.n_groups, p.key_blocks, &p.kb_chunk);
  // d = 64 fits 128 VGPRs (a few values spilled; their reloads sit after
  // the loop and, when causal, in the masked-tile pass), so two workgroups
  // share a CU; that pays once the grid has 512 workgroups, while smaller
  // grids run faster with more registers
  if constexpr (D == 64) {
    if ((int64_t)p.n_groups * p.key_blocks >= 512) {
      hipLaunchKernelGGL((bwd_dkdv_bf16<D, CAUSAL, 4>), dim3((unsigned)dkdv_grid), dim3(2 * kWaves * 64), 0, st, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((bwd_dkdv_bf16<D, CAUSAL, 2>), dim3((unsigned)dkdv_grid), dim3(2 * kWaves * 64), 0, st, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_f32_t(const BwdArgs& a) {
  F32BwdParams p;
  p.q = (const float*)a.q;
  p.k = (const float*)a.k;
  p.v = (const float*)a.v;
  p.dout = (const float*)a.dout;
  p.S = (int)a.S;
  p.S_pad = (int)pad64(a.S);
  p.H_q = a.H_q;
  p.H_kv = a.H_kv;
  p.R = a.H_q / a.H_kv;
  float* ws_lse2 = (float*)a.workspace;
  float* ws_delta = ws_lse2 + a.B * a.H_q * (int64_t)p.S_pad;
  p.ws_lse2 = ws_lse2;
  p.ws_delta = ws_delta;
  p.dq = (float*)a.dq;
  p.dk = (float*)a.dk;
  p.dv = (float*)a.dv;
  p.n_groups = (int)(a.B * a.H_kv);
  p.n_items = p.R * (int)((a.S + 31) / 32);
  p.chunks = (p.n_items + 3) / 4;
  p.key_blocks = (int)((a.S + 127) / 128);
  p.c = a.c;
  p.neg = a.negate_q ? 0x80000000u : 0u;
  p.scale = a.scale;
  hipStream_t st = (hipStream_t)a.stream;
  const int64_t nst = a.B * a.H_q * (int64_t)p.S_pad;
  hipLaunchKernelGGL((bwd_stats_f32<D>), dim3((unsigned)((nst + 255) / 256)), dim3(256), 0, st, (const float*)a.out,
                     (const float*)a.dout, a.lse, ws_lse2, ws_delta, a.B, (int)a.S, p.S_pad, a.H_q);
  hipLaunchKernelGGL((bwd_dq_f32<D, CAUSAL>), dim3((unsigned)((int64_t)p.n_groups * p.chunks)), dim3(256), 0, st, p);
  hipLaunchKernelGGL((bwd_dkdv_f32<D, CAUSAL>), dim3((unsigned)((int64_t)p.n_groups * p.key_blocks)), dim3(256), 0,
                     st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const BwdArgs& a) {
  if (a.dtype == 0) {
    switch (a.d) {
      case 32: return a.causal ? launch_bwd_bf16_t<32, true>(a) : launch_bwd_bf16_t<32, false>(a);
      case 64: return a.causal ? launch_bwd_bf16_t<64, true>(a) : launch_bwd_bf16_t<64, false>(a);
      case 128: return a.causal ? launch_bwd_bf16_t<128, true>(a) : launch_bwd_bf16_t<128, false>(a);
    }
  } else {
    switch (a.d) {
      case 32: return a.causal ? launch_bwd_f32_t<32, true>(a) : launch_bwd_f32_t<32, false>(a);
      case 64: return a.causal ? launch_bwd_f32_t<64, true>(a) : launch_bwd_f32_t<64, false>(a);
      case 128: return a.causal ? launch_bwd_f32_t<128, true>(a) : launch_bwd_f32_t<128, false>(a);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace sqa
