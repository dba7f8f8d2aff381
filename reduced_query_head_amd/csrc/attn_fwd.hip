// Decoupled-head attention forward for gfx950 (MI355X, CDNA4).
//
// Computes, for every batch b, query head h and position i,
//   out[b,i,h,:] = sum_j softmax_j(scale * <q[b,i,h,:], k[b,j,g,:]>) v[b,j,g,:]
// with g = floor(h / R), R = H_q / H_kv: the head sharing of grouped-query
// attention ("Paper explainer: GQA - Grouped-Query Attention", the GQA
// equations and the grouping figure; the PyTorch module's expand order), with
// the query-head count free as in Sparse Query Attention ("Sparse Query
// Attention (SQA)", abstract).  The softmax is evaluated online over key
// tiles (running row maximum and row sum), which equals the row-normalised
// form D(A)^-1 A V of the quantum-attention review's classical baseline
// exactly in real arithmetic.
//
// bf16 kernel design (one workgroup = WAVES waves of 64 lanes and KEYS-key
// K/V tiles: WAVES = 8 with 128-key tiles for large grids, 4 with 64-key
// tiles otherwise):
//  * A workgroup owns one key/value group (b, g) and WAVES "items"; an item
//    is 32 consecutive query positions of one query head of that group.
//    Items are ordered position-block-major, head-minor, so the waves of a
//    workgroup cover the same positions for up to WAVES heads, and every
//    K/V tile staged in LDS feeds all of them.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: keys run along M, queries along N.  Each lane
//    then holds 16 scores of a single query per 32-key block, so the row
//    maximum and row sum are in-register reductions plus one
//    v_permlane32_swap between the two lane halves.
//  * O^T = V^T P^T reuses the score accumulator as the B operand: the lane
//    that holds P[query][key] for 8 keys is exactly the lane the MFMA wants,
//    once the MFMA's K index is mapped to the keys in the order the score
//    accumulator holds them.  V^T comes from LDS with ds_read_b64_tr_b16.
//  * K and V tiles go global -> LDS directly
//    (global_load_lds_dwordx4), double-buffered, one barrier per tile.  The
//    LDS layout XOR-swizzles 16-byte chunks by the row bits so that both the
//    K operand reads and the transposed V reads are bank-conflict free.  LDS
//    operand reads run several MFMAs ahead of their use.
//  * Online softmax in the exp2 domain; the row sum adds the bf16
//    probabilities that enter the P.V product.  d = 64 and 128 without the
//    log-normaliser: the shift is the maximum of the wave's first tile and
//    stays fixed, and a range check after the key loop sends rows whose
//    probabilities or output left the fp32 range to an exact recomputation.
//    Otherwise a running maximum on every tile, moved lazily.
//  * Causal: tiles above a wave's last row are skipped, diagonal tiles are
//    masked per element; sequence tails: key rows are clamped for the loads
//    and masked in the scores, query rows past S are never stored.
//  * Grids too small to fill the chip (non-causal, d = 64: fewer than two
//    8-wave workgroups per CU) split each workgroup's key range in two or
//    four parts: waves w, w + 4, ... take the same query item, one part of
//    the keys each, and merge their running maxima, row sums and O^T
//    through LDS at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace sqa {
namespace {

using namespace dev;

constexpr int kRows = kFwdRows;   // query positions per item (one wave)
constexpr float kLazyLog2 = 8.0f;  // running-max slack before a rescale (log2 units)

struct Bf16Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int S;
  int H_q;
  int H_kv;
  int R;
  int n_groups;          // B * H_kv
  int n_items;           // R * ceil(S / kRows), items per group
  int chunks;            // ceil(n_items / items per workgroup), workgroups per group
  float c;               // |scale| * log2(e), strictly positive
  uint32_t q_sign;       // 0x8000 when scale < 0: q is negated on load (exact)
  float* lse;            // optional [B, S, H_q] row log-normaliser (natural log)
  int64_t q_stride;      // elements between consecutive positions of q (H_q * D when dense)
  int64_t kv_stride;     // same for k and v (H_kv * D when dense)
};

// Waves per SIMD the register allocation must allow: 4 for the d = 64,
// 64-key shapes of 8 waves (two workgroups per CU) and 16 waves, else 2.
template <int D, int WAVES, int KEYS>
constexpr int fwd_min_waves_per_simd() { return (D == 64 && WAVES >= 8 && KEYS == 64) ? 4 : 2; }

template <int D, bool CAUSAL, int WAVES, int KEYS, int KSPLIT>
__global__ __launch_bounds__(WAVES * 64, (fwd_min_waves_per_simd<D, WAVES, KEYS>())) void attn_fwd_bf16(Bf16Params p) {
  constexpr int KS = D / 16;      // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;      // 32-row blocks of O^T
  constexpr int NB = KEYS / 32;  // 32-key blocks per tile
  constexpr int NT = KEYS / 16;  // 16-key MFMA steps of P.V per tile
  constexpr int TILE = KEYS * D; // elements per tile
  constexpr int IPW = WAVES / KSPLIT;  // items per workgroup
  static_assert(KSPLIT == 1 || ((KSPLIT == 2 || KSPLIT == 4) && IPW == 4 && KEYS == 64),
                "key split: two or four parts of four waves, 64-key tiles");
  // one tile per key part in each buffer
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k0[KSPLIT * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k1[KSPLIT * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v0[KSPLIT * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v1[KSPLIT * TILE];

  const int lane = threadIdx.x & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // with a key split, waves w, w + IPW, ... take the same query item and the
  // two halves of the workgroup's key range (merged at the end)
  const int wave = KSPLIT == 1 ? wave_id : wave_id % IPW;
  const int kpart = KSPLIT == 1 ? 0 : wave_id / IPW;
  const int half = lane >> 5;     // which half of the wave
  const int col = lane & 31;      // query column of this lane in S^T / O^T
  const int S = p.S;

  // workgroup -> (group, chunk).  Consecutive workgroups cycle through the
  // groups, so with round-robin dispatch over the XCDs each XCD keeps
  // streaming the same groups' K/V; causal chunks go heaviest first.
  const int grp = blockIdx.x % p.n_groups;
  const int ord = blockIdx.x / p.n_groups;
  const int chunk = CAUSAL ? (p.chunks - 1 - ord) : ord;
  const int b = grp / p.H_kv;
  const int g = grp % p.H_kv;

  const int item = chunk * IPW + wave;
  const bool active = item < p.n_items;
  const int pos0 = (item / p.R) * kRows;
  const int h = g * p.R + item % p.R;

  const int last_item = min(chunk * IPW + IPW - 1, p.n_items - 1);
  const int wg_last_pos = min((last_item / p.R) * kRows + kRows - 1, S - 1);
  const int wg_tiles = CAUSAL ? wg_last_pos / KEYS + 1 : (S + KEYS - 1) / KEYS;
  // this wave's key part: tiles [t_first, t_first + n_tiles) of the
  // workgroup's range; every wave runs part_steps steps (one barrier each)
  const int part_steps = (wg_tiles + KSPLIT - 1) / KSPLIT;
  const int t_first = kpart * part_steps;
  const int n_tiles = KSPLIT == 1 ? wg_tiles : max(0, min(wg_tiles - t_first, part_steps));

  const int64_t kv_stride = p.kv_stride;
  const uint16_t* k_base = p.k + (int64_t)b * S * kv_stride + g * D + (int64_t)t_first * KEYS * kv_stride;
  const uint16_t* v_base = p.v + (int64_t)b * S * kv_stride + g * D + (int64_t)t_first * KEYS * kv_stride;
  const int S_part = S - t_first * KEYS;   // keys from this part's first tile to the end

  TileCopy<D, IPW, KEYS> cp;
  cp.init(kv_stride, wave, lane);
  // first K/V tile in flight while Q loads
  if (KSPLIT == 1 || n_tiles > 0) {
    cp.issue(k_base, kv_stride, S_part, (SQA_LDS uint16_t*)lds_k0 + kpart * TILE, wave);
    cp.issue(v_base, kv_stride, S_part, (SQA_LDS uint16_t*)lds_v0 + kpart * TILE, wave);
  }

  // Q^T as the B operand: lane holds query (pos0 + col), head dims
  // ks*16 + half*8 ... +7.
  bf16x8 qf[KS];
  {
    const int qrow = min(pos0 + col, S - 1);
    const uint16_t* qp = p.q + ((int64_t)b * S + qrow) * p.q_stride + h * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = *(const u32x4*)(qp + ks * 16);
      const uint32_t sgn = p.q_sign * 0x10001u;
      raw ^= (u32x4){sgn, sgn, sgn, sgn};
      qf[ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // per-lane LDS element offsets (tile-relative), independent of the tile
  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = kpart * TILE + tile_off<D>(col, ks * 16 + half * 8);
  // transposed V reads: lane (within its 16-lane group) supplies the address
  // of row e = (lane%16)/4 and columns 4*(lane%4) ... +3 of a 4 x 16 block;
  // the hardware returns to lane i the 4 rows of column i.
  int v_off[DB][2];
  {
    const int grp16 = lane >> 4, i16 = lane & 15, e = i16 >> 2, c4 = i16 & 3;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 4 * half + 8 * j + e;
        const int cc = db * 32 + (grp16 & 1) * 16 + 4 * c4;
        v_off[db][j] = kpart * TILE + tile_off<D>(row, cc);
      }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  // Row sums on the matrix cores (d = 128, and the non-causal 8-wave d = 64
  // shape, whose register budget allows it): per P.V step one
  // v_mfma_f32_16x16x32_bf16 takes the bf16 probabilities as its B operand
  // (lane l supplies column l % 16, k-group l / 16, i.e. query l % 32 and key
  // half l / 32) and a 0/1 A operand that, for output rows 0-7, selects the
  // k-groups of queries 0-15 and, for rows 8-15, those of queries 16-31.
  // Every output row then holds, per column n, the sum over the step's 16
  // keys of query n (rows 0-7) or n + 16 (rows 8-15), accumulated over the
  // whole key loop.  This replaces four v_dot2 per step (32 VALU
  // instructions per 128-key tile) with one short MFMA; measured 0.2-0.8 %
  // faster on the 32K-200K workloads and 3-4 % at d = 64 (S = 4096 and 32K,
  // non-causal), where the softmax's VALU work is the tighter bound.
  constexpr bool ROWMFMA = D == 128 || (D == 64 && !CAUSAL && WAVES >= 8);
  // d = 64 and 128 without the log-normaliser: the softmax shift is the
  // maximum of the wave's first tile and stays fixed (no maximum on later
  // tiles; 3-4 % faster at d = 128, up to 5 % at d = 64).  d = 32 keeps a
  // running maximum on every tile: there the fixed shift's range check took
  // a register past the 4-waves-per-SIMD budget.
  constexpr bool FIXED_SHIFT = D >= 64;
  f32x4 lsum = (f32x4){0.f, 0.f, 0.f, 0.f};
  bf16x8 rs_sel;
  {
    const __bf16 one = (((lane >> 4) & 1) == ((lane & 15) >> 3)) ? (__bf16)1.0f : (__bf16)0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) rs_sel[e] = one;
  }
  // lane l accumulates the row sum of the query of lane l ^ 16 for
  // 16 <= l < 48, of its own query otherwise
  const int rs_src = (lane >= 16 && lane < 48) ? (lane ^ 16) : lane;
  // with the log-normaliser requested, the running maximum: its dominant
  // probabilities are then close to 1 and exact in bf16, which the log of
  // the row sum needs (with a fixed shift a dominant p keeps an arbitrary
  // mantissa, whose bf16 rounding, up to 2^-8, goes into ln l unchanged)
  const bool track_max = p.lse != nullptr;
  const float c = p.c;
  const int my_q = pos0 + col;
  const int wave_last = pos0 + kRows - 1;

  auto step = [&](int t, SQA_LDS uint16_t* kt_cur, SQA_LDS uint16_t* vt_cur, SQA_LDS uint16_t* kt_nxt, SQA_LDS uint16_t* vt_nxt,
                  bool first) {
    const int kv0l = t * KEYS;                // first key of the tile within the part
    const int kv0 = t_first * KEYS + kv0l;    // and within the sequence
    wait_copies();     // this wave's copies of tile t landed
    __syncthreads();   // everyone's copies landed; tile t-1 fully consumed
    // copies of tile t+1 into the other buffers; issued after this tile's
    // K.Q^T MFMAs so that their issue overlaps matrix work
    auto copy_next = [&]() {
      if (t + 1 < n_tiles) {
        const int64_t nxt = (int64_t)(kv0l + KEYS) * kv_stride;
        cp.issue(k_base + nxt, kv_stride, S_part - kv0l - KEYS, kt_nxt + kpart * TILE, wave);
        cp.issue(v_base + nxt, kv_stride, S_part - kv0l - KEYS, vt_nxt + kpart * TILE, wave);
      }
    };
    if ((KSPLIT > 1 && t >= n_tiles) || !active || (CAUSAL && kv0 > wave_last)) {  // no work on this tile
      copy_next();
      return;
    }

    const SQA_LDS uint16_t* kt = kt_cur;
    const SQA_LDS uint16_t* vt = vt_cur;

    // S^T = K Q^T
    f32x16 s[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 a = *(const SQA_LDS bf16x8*)(kt + nb * 32 * D + k_off[ks]);
        s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[nb], 0, 0, 0);
      }
    lds_mfma_pipeline_hint<KS * NB, 1, 4>();
    copy_next();

    // mask: key index of s[nb][r] is kv0 + 4*half + (nb*32 + 8*(r/4) + r%4)
    const bool need_mask = (kv0 + KEYS > S) || (CAUSAL && kv0 + KEYS - 1 > pos0);
    if (need_mask) {
      const int lim = (CAUSAL ? min(my_q, S - 1) : S - 1) - kv0 - 4 * half;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (nb * 32 + 8 * (r >> 2) + (r & 3) > lim) s[nb][r] = -__builtin_inff();
    }

    // online softmax in the exp2 domain: p = 2^(c*s - m); the result is the
    // same for any shift m (it cancels in the final division by the row
    // sum), which only has to keep p and O in range.  Fixed shift: m is the
    // maximum of the wave's first tile (every row sees a key there) and stays
    // fixed; a later score far above it could overflow p or O, which the
    // range check after the key loop catches, and the rows are then
    // recomputed with a running maximum.
    if (FIXED_SHIFT && !track_max) {
      if (first) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][r]);
        mx = wave_pair_max(mx);
        m_run = mx > -__builtin_inff() ? mx * c : 0.f;
      }
    } else {
      // running maximum on every tile, moved only when a row's maximum
      // exceeds it by more than kLazyLog2 (then p <= 2^kLazyLog2)
      float mx = -__builtin_inff();
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][r]);
      mx = wave_pair_max(mx);
      const float m_cand = mx * c;
      const bool grow = m_cand > m_run + kLazyLog2;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? m_cand : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        if constexpr (ROWMFMA) {
          const float a_rs = __int_as_float(__builtin_amdgcn_ds_bpermute(rs_src * 4, __float_as_int(alpha)));
          lsum *= a_rs;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
    }
    // From the exponentials to the last P.V MFMA this wave issues ahead of
    // the other wave on its SIMD (which is then in its K.Q^T or maximum
    // phase): measured 1-2 % faster at d = 128 and 2-7 % at d = 64, with the
    // same results.  With 8 waves at d = 128 the two waves of a SIMD (w and
    // w + 4) take different levels, so that when both are in this phase one
    // of them drains its P.V chain first instead of the two interleaving:
    // a further 1.0-1.3 % at d = 128; at d = 64 (4 waves per SIMD) it cost
    // 2-3 %, so that shape keeps one level.
    if (WAVES == 8 && D == 128 && wave_id < WAVES / 2)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(2);
    const float neg_m = -m_run;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][r], c, neg_m));

    // O^T += V^T P^T, 16 keys per MFMA.  MFMA k-slot half*8 + e maps to key
    // 16*(step%2) + 4*half + e (e < 4) or + 8 + 4*half + (e-4) of block step/2,
    // which is where the score accumulator left them.
    // the row sum adds the bf16 probabilities the MFMA multiplies, two per
    // v_dot2 (fp32 accumulation)
    float psum = 0.f;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int st = 0; st < NT; ++st) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[st >> 1][(st & 1) * 8 + e];
      if constexpr (ROWMFMA) {
        lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rs_sel, pb, lsum, 0, 0, 0);
      } else {
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          psum = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pb[e], pb[e + 1]}, ones, psum, false);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (SQA_LDS bf16x4*)(vt + st * 16 * D + v_off[db][0]));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (SQA_LDS bf16x4*)(vt + st * 16 * D + v_off[db][1]));
        const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
      }
    }
    lds_mfma_pipeline_hint<NT * (DB + (ROWMFMA ? 1 : 0)), 2, 4>();
    __builtin_amdgcn_s_setprio(0);
    if constexpr (!ROWMFMA) l_run += psum;
  };
  const int steps = KSPLIT == 1 ? n_tiles : part_steps;
  SQA_LDS uint16_t* const k0b = (SQA_LDS uint16_t*)lds_k0;
  SQA_LDS uint16_t* const v0b = (SQA_LDS uint16_t*)lds_v0;
  SQA_LDS uint16_t* const k1b = (SQA_LDS uint16_t*)lds_k1;
  SQA_LDS uint16_t* const v1b = (SQA_LDS uint16_t*)lds_v1;
  if constexpr (FIXED_SHIFT) {
    // the first tile (which takes the maximum) peeled off the loop
    if (steps > 0) step(0, k0b, v0b, k1b, v1b, true);
    for (int t = 1; t < steps; t += 2) {
      step(t, k1b, v1b, k0b, v0b, false);
      if (t + 1 < steps) step(t + 1, k0b, v0b, k1b, v1b, false);
    }
  } else {
    for (int t = 0; t < steps; t += 2) {
      step(t, k0b, v0b, k1b, v1b, false);
      if (t + 1 < steps) step(t + 1, k1b, v1b, k0b, v0b, false);
    }
  }

  if constexpr (ROWMFMA) {
    // move each query's row sum to its own lanes (lanes 16-31 and 32-47
    // swap) while every lane of the wave is active; the two lanes of a query
    // each keep half of it (exact), as the v_dot2 path's partial sums
    const int src = (lane >= 16 && lane < 48) ? (lane ^ 48) : lane;
    l_run = 0.5f * __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(lsum[0])));
  }

  // Range check (fixed shift).  The first tile's maximum contributes p = 1,
  // so the row sum is at least 1 unless that tile showed the row no key;
  // every p is at most the row sum, so a sum of at most 2^64 and a finite O
  // mean that no p or product overflowed.  Otherwise the wave recomputes its
  // rows over its key range from global memory, 32 keys at a time with a
  // running maximum (no barrier: the other waves go on).
  if (FIXED_SHIFT && !track_max && active) {
    const float l_pair = wave_pair_sum(l_run);
    bool ok = l_pair >= 0.5f && l_pair <= 0x1p64f;   // false for NaN
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) ok = ok && __builtin_fabsf(o[db][r]) < __builtin_inff();
    if (__builtin_amdgcn_ballot_w64(!ok)) {
      const int key_lo = t_first * KEYS;
      const int key_hi = CAUSAL ? min(S, wave_last + 1) : min(S, (t_first + n_tiles) * KEYS);
      const int last_key = min(CAUSAL ? min(my_q, S - 1) : S - 1, key_hi - 1);
      const uint16_t* kg = p.k + (int64_t)b * S * kv_stride + g * D + half * 8;
      const uint16_t* vg = p.v + (int64_t)b * S * kv_stride + g * D + col;
      m_run = -__builtin_inff();
      l_run = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
      for (int k0 = key_lo; k0 < key_hi; k0 += 32) {
        // S^T block: key k0 + 8*(r/4) + 4*half + r%4 in register r
        f32x16 sb = (f32x16){};
        const uint16_t* kp = kg + (int64_t)min(k0 + col, S - 1) * kv_stride;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kp + ks * 16), qf[ks], sb, 0, 0, 0);
        const int lim = last_key - k0 - 4 * half;
        float mx = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (8 * (r >> 2) + (r & 3) > lim) sb[r] = -__builtin_inff();
          mx = fmaxf(mx, sb[r]);
        }
        mx = wave_pair_max(mx);
        // a lane that has seen no visible key yet keeps m = -inf and adds zeros
        const float m_new = fmaxf(m_run, mx * c);
        const bool seen = m_new > -__builtin_inff();
        const float alpha = seen ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        const float neg_m = seen ? -m_new : 0.f;
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        // P rounded to bf16, the row sum over the rounded values (as in the
        // tile loop); O^T += V^T P^T with k-slot half*8 + e of step st at key
        // k0 + 16*st + 4*half + e (e < 4) or k0 + 16*st + 8 + 4*half + e - 4
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pb[e] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sb[st * 8 + e], c, neg_m));
            l_run += (float)pb[e];
          }
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            bf16x8 va;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int key = min(k0 + 16 * st + (e < 4 ? 4 * half + e : 8 + 4 * half + e - 4), S - 1);
              va[e] = __builtin_bit_cast(__bf16, vg[(int64_t)key * kv_stride + db * 32]);
            }
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
          }
        }
      }
    }
  }

  if constexpr (KSPLIT > 1) {
    // merge the key parts of each item: parts 1 .. KSPLIT-1 hand their
    // running maxima, row sums and unnormalised O^T to part 0 through LDS
    // (the tile buffers, free once every wave is past its last tile); part
    // 0 rescales all of them to the largest maximum and adds them in part
    // order (a part with no visible key holds m = -inf, l = 0, O = 0 and adds
    // nothing; part 0 always sees key 0).
    // O^T slots of DB*16*64 floats: with two parts, items 0, 1 use lds_k0
    // and items 2, 3 lds_k1, the statistics lds_v0; with four parts, part p
    // uses lds_k0, lds_k1, lds_v0 for p = 1, 2, 3 (one slot per item), the
    // statistics lds_v1 ([KSPLIT-1][IPW][2][64] floats).
    constexpr int OX = DB * 16 * 64;
    static_assert((KSPLIT == 2 ? 2 : IPW) * OX * 4 <= KSPLIT * TILE * 2, "O exchange fits the tile buffers");
    auto xo_slot = [&](int part) -> SQA_LDS float* {
      if constexpr (KSPLIT == 2)
        return (SQA_LDS float*)(wave < 2 ? (SQA_LDS uint16_t*)lds_k0 : (SQA_LDS uint16_t*)lds_k1) + (wave & 1) * OX;
      else
        return (SQA_LDS float*)(part == 1   ? (SQA_LDS uint16_t*)lds_k0
                                : part == 2 ? (SQA_LDS uint16_t*)lds_k1
                                            : (SQA_LDS uint16_t*)lds_v0) + wave * OX;
    };
    SQA_LDS float* xm = (SQA_LDS float*)(KSPLIT == 2 ? (SQA_LDS uint16_t*)lds_v0 : (SQA_LDS uint16_t*)lds_v1);
    wait_copies();
    __syncthreads();
    if (kpart > 0 && active) {
      SQA_LDS float* xo = xo_slot(kpart);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(db * 16 + r) * 64 + lane] = o[db][r];
      xm[(((kpart - 1) * IPW + wave) * 2) * 64 + lane] = m_run;
      xm[(((kpart - 1) * IPW + wave) * 2 + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    if (kpart > 0) return;
    if (active) {
      // one part at a time: rescale to the larger maximum and add
#pragma unroll
      for (int j = 0; j < KSPLIT - 1; ++j) {
        const float mj = xm[((j * IPW + wave) * 2) * 64 + lane];
        const float lj = xm[((j * IPW + wave) * 2 + 1) * 64 + lane];
        const SQA_LDS float* xo = xo_slot(j + 1);
        const float m_new = fmaxf(m_run, mj);
        const float a0 = __builtin_amdgcn_exp2f(m_run - m_new);
        const float a1 = __builtin_amdgcn_exp2f(mj - m_new);
        l_run = l_run * a0 + lj * a1;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * a0 + xo[(db * 16 + r) * 64 + lane] * a1;
          // each part's reads stay after the previous part's sums (hoisted
          // together they spilled)
          asm volatile("" : "+v"(o[db]));
        }
        m_run = m_new;
      }
    }
  }

  if (!active) return;
  const int out_pos = pos0 + col;
  if (out_pos >= S) return;  // lanes l and l^32 share out_pos, so pairs leave together
  const float l_tot = wave_pair_sum(l_run);
  const float inv = 1.0f / l_tot;
  // log of the row normaliser: scores entered the softmax as s*c with
  // c = scale*log2(e), so ln(sum_j exp(scale*s_j)) = ln2 * (m + log2(l))
  if (p.lse && half == 0) p.lse[((int64_t)b * S + out_pos) * p.H_q + h] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
  uint16_t* op = p.o + (((int64_t)b * S + out_pos) * p.H_q + h) * D;
  // O^T[db] register r holds head dim db*32 + 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[db][4 * j + e] * inv);
      *(bf16x4*)(op + db * 32 + 8 * j + 4 * half) = w;
    }
}

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;            // optional [B, S, H_q] row log-normaliser (natural log)
  int S;
  int H_q;
  int H_kv;
  int R;
  int n_groups;          // B * H_kv
  int n_items;           // R * ceil(S / 32), items per group
  int chunks;            // ceil(n_items / 4), workgroups per group
  float c;               // |scale| * log2(e), strictly positive
  uint32_t q_sign;       // 0x80000000 when scale < 0: q is negated on load (exact)
  int64_t q_stride;      // elements between consecutive positions of q
  int64_t kv_stride;     // same for k and v
};

// fp32 path on the matrix cores: v_mfma_f32_32x32x2_f32 (fp32 operands and
// accumulation) for both products, the same transposed formulation as the
// bf16 kernel (S^T = K Q^T with keys along M; O^T += V^T P^T with the score
// accumulator as the P operand, in fp32).  A workgroup of 4 waves owns one
// K/V group and 4 items of 32 query positions (position-major, head-minor);
// 32-key K and V tiles are staged in LDS through registers with rows padded
// by one float (the K operand reads a column: 32 rows at one dim), double
// buffered with the next-but-one tile's loads in flight.  Each wave holds its
// Q^T operand (D/2 floats per lane) for the whole key loop.  The softmax is
// the bf16 kernel's (exp2 domain, lazily moved running maximum), with the
// probabilities kept in fp32.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fwd_f32(F32Params p) {
  constexpr int WAVES = 4;
  constexpr int KP = D / 2;   // MFMA k-steps over the head dimension (two dims each)
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int KB = 32;      // keys per tile
  constexpr int LD = F32Tile<D>::LD;   // LDS row stride in floats
  __shared__ float lds_k[2][KB * LD];
  __shared__ float lds_v[2][KB * LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  const int S = p.S;

  // workgroup -> (group, chunk) as in the bf16 kernel; causal heaviest first
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

  // K and V tiles through registers (rows past S clamped, masked in the scores)
  const float* k_base = p.k + (int64_t)b * S * p.kv_stride + g * D;
  const float* v_base = p.v + (int64_t)b * S * p.kv_stride + g * D;
  F32Tile<D> tk, tv;
  tk.load(k_base, p.kv_stride, 0, S, tid);
  tv.load(v_base, p.kv_stride, 0, S, tid);

  // Q^T as the B operand: lane holds query pos0 + col, dims 2*ks + half
  float qf[KP];
  {
    const int qrow = min(pos0 + col, S - 1);
    const float* qp = p.q + ((int64_t)b * S + qrow) * p.q_stride + h * D + half;
#pragma unroll
    for (int ks = 0; ks < KP; ++ks) qf[ks] = __uint_as_float(__float_as_uint(qp[2 * ks]) ^ p.q_sign);
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float c = p.c;
  const int my_q = pos0 + col;
  const int wave_last = pos0 + 31;

  tk.store(lds_k[0], tid);
  tv.store(lds_v[0], tid);
  if (n_tiles > 1) {
    tk.load(k_base, p.kv_stride, KB, S, tid);
    tv.load(v_base, p.kv_stride, KB, S, tid);
  }
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    __syncthreads();   // tile t stored by everyone; tile t-1 fully consumed
    if (t + 1 < n_tiles) {
      tk.store(lds_k[buf ^ 1], tid);
      tv.store(lds_v[buf ^ 1], tid);
    }
    if (t + 2 < n_tiles) {
      tk.load(k_base, p.kv_stride, (t + 2) * KB, S, tid);
      tv.load(v_base, p.kv_stride, (t + 2) * KB, S, tid);
    }
    const int kv0 = t * KB;
    if (!active || (CAUSAL && kv0 > wave_last)) continue;
    const float* kt = lds_k[buf];
    const float* vt = lds_v[buf];

    // S^T = K Q^T: A operand K[key col][dim 2*ks + half]
    f32x16 s = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KP; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kt[col * LD + 2 * ks + half], qf[ks], s, 0, 0, 0);

    // mask: s[r] holds key kv0 + 8*(r/4) + 4*half + r%4
    if ((kv0 + KB > S) || (CAUSAL && kv0 + KB - 1 > pos0)) {
      const int lim = (CAUSAL ? min(my_q, S - 1) : S - 1) - kv0 - 4 * half;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) > lim) s[r] = -__builtin_inff();
    }

    float mx = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = wave_pair_max(mx);
    const float m_cand = mx * c;
    const bool grow = m_cand > m_run + kLazyLog2;
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
    for (int r = 0; r < 16; ++r) {
      s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, neg_m));
      l_run += s[r];
    }

    // O^T += V^T P^T: score register r supplies the key pair
    // 8*(r/4) + r%4 (k = 0, lanes 0-31) and that + 4 (k = 1, lanes 32-63)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * half + (r & 3);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vt[key * LD + db * 32 + col], s[r], o[db], 0, 0, 0);
    }
  }

  if (!active) return;
  const int out_pos = pos0 + col;
  if (out_pos >= S) return;  // lanes l and l^32 share out_pos, so pairs leave together
  const float l_tot = wave_pair_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (p.lse && half == 0) p.lse[((int64_t)b * S + out_pos) * p.H_q + h] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
  float* op = p.o + (((int64_t)b * S + out_pos) * p.H_q + h) * D;
  // O^T[db] register r holds head dim db*32 + 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(f32x4*)(op + db * 32 + 8 * j + 4 * half) =
          (f32x4){o[db][4 * j] * inv, o[db][4 * j + 1] * inv, o[db][4 * j + 2] * inv, o[db][4 * j + 3] * inv};
}



template <int D, bool CAUSAL, int WAVES, int KEYS, int KSPLIT = 1>
hipError_t launch_bf16_w(const LaunchArgs& a) {
  Bf16Params p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.o = (uint16_t*)a.out;
  p.S = (int)a.S;
  p.H_q = a.H_q;
  p.H_kv = a.H_kv;
  p.R = a.H_q / a.H_kv;
  p.n_groups = (int)(a.B * a.H_kv);
  const int n_pos_blocks = (int)((a.S + kRows - 1) / kRows);
  p.n_items = p.R * n_pos_blocks;
  p.chunks = (p.n_items + WAVES / KSPLIT - 1) / (WAVES / KSPLIT);
  p.c = a.c;
  p.q_sign = a.negate_q ? 0x8000u : 0u;
  p.lse = a.lse;
  p.q_stride = a.q_stride;
  p.kv_stride = a.kv_stride;
  const int64_t grid = (int64_t)p.n_groups * p.chunks;
  hipLaunchKernelGGL((attn_fwd_bf16<D, CAUSAL, WAVES, KEYS, KSPLIT>), dim3((unsigned)grid), dim3(WAVES * 64), 0,
                     (hipStream_t)a.stream, p);
  return hipGetLastError();
}

constexpr int kCUs = 256;

// Workgroup shape per head dim, when the grid of 8-wave workgroups still
// fills the chip (else 4 waves and 64-key tiles, twice the workgroups):
// - d = 128: 8 waves, 128-key tiles; 231 VGPRs, so one workgroup per CU
//   (2 waves per SIMD); taken from 512 workgroups on.
// - d = 64: 8 waves, 64-key tiles, held to 128 VGPRs so that two workgroups
//   share a CU (4 waves per SIMD); taken from 512 workgroups on.  Measured
//   1.5-7 % faster than 128-key tiles at 2 waves per SIMD.  Non-causal
//   grids of 129-511 such workgroups split the key range in two (twice the
//   workgroups): at S = 4096, B = 2, the 8/4 heads went from 0.0789 to
//   0.0764 ms.  Smaller non-causal grids split it in four, with 16-wave
//   workgroups (four items, 128 KiB of LDS, one per CU at 4 waves per
//   SIMD).  The 4/4 heads at S = 4096, B = 2 (128 such workgroups): 0.0544
//   ms unsplit, 0.0430 ms split in two (one box); on another box 0.0422 ms
//   split in two, 0.0400 ms split in four, and 0.0406 ms split in two with
//   a third tile buffer (LDS allows it at one workgroup per CU).
// - d = 32: 8 waves, 128-key tiles (126 VGPRs, two workgroups per CU); taken
//   from 512 workgroups on.  2-5 % faster than the 4-wave shape.
template <int D, bool CAUSAL>
hipError_t launch_bf16_t(const LaunchArgs& a) {
  const int64_t items = (int64_t)(a.H_q / a.H_kv) * ((a.S + kRows - 1) / kRows);
  const int64_t wgs8 = a.B * a.H_kv * ((items + 7) / 8);
  if constexpr (D == 64) {
    if (wgs8 >= 2 * kCUs) return launch_bf16_w<D, CAUSAL, 8, 64>(a);
    if constexpr (!CAUSAL) {
      if (wgs8 * 2 > kCUs) return launch_bf16_w<D, CAUSAL, 8, 64, 2>(a);
      return launch_bf16_w<D, CAUSAL, 16, 64, 4>(a);
    }
  } else {
    if (wgs8 >= 2 * kCUs) return launch_bf16_w<D, CAUSAL, 8, 128>(a);
  }
  return launch_bf16_w<D, CAUSAL, 4, 64>(a);
}

template <int D, bool CAUSAL>
hipError_t launch_f32_t(const LaunchArgs& a) {
  F32Params p;
  p.q = (const float*)a.q;
  p.k = (const float*)a.k;
  p.v = (const float*)a.v;
  p.o = (float*)a.out;
  p.lse = a.lse;
  p.S = (int)a.S;
  p.H_q = a.H_q;
  p.H_kv = a.H_kv;
  p.R = a.H_q / a.H_kv;
  p.n_groups = (int)(a.B * a.H_kv);
  p.n_items = p.R * (int)((a.S + 31) / 32);
  p.chunks = (p.n_items + 3) / 4;
  p.c = a.c;
  p.q_sign = a.negate_q ? 0x80000000u : 0u;
  p.q_stride = a.q_stride;
  p.kv_stride = a.kv_stride;
  const int64_t grid = (int64_t)p.n_groups * p.chunks;
  hipLaunchKernelGGL((attn_fwd_f32<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, (hipStream_t)a.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const LaunchArgs& a) {
  if (a.dtype == 0) {
    switch (a.d) {
      case 32: return a.causal ? launch_bf16_t<32, true>(a) : launch_bf16_t<32, false>(a);
      case 64: return a.causal ? launch_bf16_t<64, true>(a) : launch_bf16_t<64, false>(a);
      case 128: return a.causal ? launch_bf16_t<128, true>(a) : launch_bf16_t<128, false>(a);
    }
  } else {
    switch (a.d) {
      case 32: return a.causal ? launch_f32_t<32, true>(a) : launch_f32_t<32, false>(a);
      case 64: return a.causal ? launch_f32_t<64, true>(a) : launch_f32_t<64, false>(a);
      case 128: return a.causal ? launch_f32_t<128, true>(a) : launch_f32_t<128, false>(a);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace sqa
