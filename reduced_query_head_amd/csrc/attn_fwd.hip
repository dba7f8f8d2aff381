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
//  * Online softmax in the exp2 domain with a lazily moved running maximum;
//    the row sum adds the bf16 probabilities that enter the P.V product.
//  * Causal: tiles above a wave's last row are skipped, diagonal tiles are
//    masked per element; sequence tails: key rows are clamped for the loads
//    and masked in the scores, query rows past S are never stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace sqa {
namespace {

using namespace dev;

constexpr int kRows = 32;         // query positions per item (one wave)
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
  int chunks;            // ceil(n_items / WAVES), workgroups per group
  float c;               // |scale| * log2(e), strictly positive
  uint32_t q_sign;       // 0x8000 when scale < 0: q is negated on load (exact)
  float* lse;            // optional [B, S, H_q] row log-normaliser (natural log)
  int64_t q_stride;      // elements between consecutive positions of q (H_q * D when dense)
  int64_t kv_stride;     // same for k and v (H_kv * D when dense)
};

// Waves per SIMD the register allocation must allow: 4 for the d = 64,
// 8-wave, 64-key shape (two workgroups per CU), else 2.
template <int D, int WAVES, int KEYS>
constexpr int fwd_min_waves_per_simd() { return (D == 64 && WAVES == 8 && KEYS == 64) ? 4 : 2; }

template <int D, bool CAUSAL, int WAVES, int KEYS>
__global__ __launch_bounds__(WAVES * 64, (fwd_min_waves_per_simd<D, WAVES, KEYS>())) void attn_fwd_bf16(Bf16Params p) {
  constexpr int KS = D / 16;      // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;      // 32-row blocks of O^T
  constexpr int NB = KEYS / 32;  // 32-key blocks per tile
  constexpr int NT = KEYS / 16;  // 16-key MFMA steps of P.V per tile
  constexpr int TILE = KEYS * D; // elements per tile
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v1[TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

  const int item = chunk * WAVES + wave;
  const bool active = item < p.n_items;
  const int pos0 = (item / p.R) * kRows;
  const int h = g * p.R + item % p.R;

  const int last_item = min(chunk * WAVES + WAVES - 1, p.n_items - 1);
  const int wg_last_pos = min((last_item / p.R) * kRows + kRows - 1, S - 1);
  const int n_tiles = CAUSAL ? wg_last_pos / KEYS + 1 : (S + KEYS - 1) / KEYS;

  const int64_t kv_stride = p.kv_stride;
  const uint16_t* k_base = p.k + (int64_t)b * S * kv_stride + g * D;
  const uint16_t* v_base = p.v + (int64_t)b * S * kv_stride + g * D;

  TileCopy<D, WAVES, KEYS> cp;
  cp.init(kv_stride, wave, lane);
  // first K/V tile in flight while Q loads
  cp.issue(k_base, kv_stride, S, (SQA_LDS uint16_t*)lds_k0, wave);
  cp.issue(v_base, kv_stride, S, (SQA_LDS uint16_t*)lds_v0, wave);

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
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = tile_off<D>(col, ks * 16 + half * 8);
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
        v_off[db][j] = tile_off<D>(row, cc);
      }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float c = p.c;
  const int my_q = pos0 + col;
  const int wave_last = pos0 + kRows - 1;

  auto step = [&](int t, SQA_LDS uint16_t* kt_cur, SQA_LDS uint16_t* vt_cur, SQA_LDS uint16_t* kt_nxt, SQA_LDS uint16_t* vt_nxt) {
    const int kv0 = t * KEYS;
    wait_copies();     // this wave's copies of tile t landed
    __syncthreads();   // everyone's copies landed; tile t-1 fully consumed
    // copies of tile t+1 into the other buffers; issued after this tile's
    // K.Q^T MFMAs so that their issue overlaps matrix work
    auto copy_next = [&]() {
      if (t + 1 < n_tiles) {
        const int64_t nxt = (int64_t)(kv0 + KEYS) * kv_stride;
        cp.issue(k_base + nxt, kv_stride, S - kv0 - KEYS, kt_nxt, wave);
        cp.issue(v_base + nxt, kv_stride, S - kv0 - KEYS, vt_nxt, wave);
      }
    };
    if (!active || (CAUSAL && kv0 > wave_last)) {  // no work on this tile
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

    // online softmax in the exp2 domain: p = 2^(c*s - m).  The running max m
    // is only moved when a row's maximum grows by more than 2^kLazyLog2, so
    // p <= 2^kLazyLog2 and the accumulator is rarely rescaled; the result is
    // the same for any m (it cancels in the final division by the row sum).
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
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    // From the exponentials to the last P.V MFMA this wave issues ahead of
    // the other wave on its SIMD (which is then in its K.Q^T or maximum
    // phase): measured 1-2 % faster at d = 128 and 2-7 % at d = 64, with the
    // same results.
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
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        psum = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){pb[e], pb[e + 1]}, ones, psum, false);
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
    lds_mfma_pipeline_hint<NT * DB, 2, 4>();
    __builtin_amdgcn_s_setprio(0);
    l_run += psum;
  };
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, (SQA_LDS uint16_t*)lds_k0, (SQA_LDS uint16_t*)lds_v0, (SQA_LDS uint16_t*)lds_k1, (SQA_LDS uint16_t*)lds_v1);
    if (t + 1 < n_tiles) step(t + 1, (SQA_LDS uint16_t*)lds_k1, (SQA_LDS uint16_t*)lds_v1, (SQA_LDS uint16_t*)lds_k0, (SQA_LDS uint16_t*)lds_v0);
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

// fp32 path: one thread per (b, position, head), online softmax over keys in
// fp32.  Plain VALU arithmetic; meant for exactness checks at small sizes.
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32(const float* __restrict__ q,
                                                    const float* __restrict__ k,
                                                    const float* __restrict__ v, float* __restrict__ o,
                                                    float* __restrict__ lse, int64_t B, int S, int H_q,
                                                    int H_kv, int R, float c, int causal) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= B * S * H_q) return;
  const int h = (int)(t % H_q);
  const int i = (int)((t / H_q) % S);
  const int64_t b = t / ((int64_t)H_q * S);
  const int g = h / R;
  float qv[D], acc[D];
  const float* qp = q + t * D;
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = qp[e];
    acc[e] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;
  const int last = causal ? i : S - 1;
  for (int j = 0; j <= last; ++j) {
    const float* kp = k + ((b * S + j) * H_kv + g) * D;
    const float* vp = v + ((b * S + j) * H_kv + g) * D;
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
  if (lse) lse[t] = (m + log2f(l)) * 0.69314718055994531f;
  float* op = o + t * D;
#pragma unroll
  for (int e = 0; e < D; ++e) op[e] = acc[e] * inv;
}



template <int D, bool CAUSAL, int WAVES, int KEYS>
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
  p.chunks = (p.n_items + WAVES - 1) / WAVES;
  p.c = a.c;
  p.q_sign = a.negate_q ? 0x8000u : 0u;
  p.lse = a.lse;
  p.q_stride = a.q_stride;
  p.kv_stride = a.kv_stride;
  const int64_t grid = (int64_t)p.n_groups * p.chunks;
  hipLaunchKernelGGL((attn_fwd_bf16<D, CAUSAL, WAVES, KEYS>), dim3((unsigned)grid), dim3(WAVES * 64), 0,
                     (hipStream_t)a.stream, p);
  return hipGetLastError();
}

constexpr int kCUs = 256;

// Workgroup shape per head dim, when the grid of 8-wave workgroups still
// fills the chip (else 4 waves and 64-key tiles, twice the workgroups):
// - d = 128: 8 waves, 128-key tiles; 231 VGPRs, so one workgroup per CU
//   (2 waves per SIMD); taken from 512 workgroups on.
// - d = 64: 8 waves, 64-key tiles, held to 128 VGPRs so that two workgroups
//   share a CU (4 waves per SIMD); taken from 256 workgroups on.  Measured
//   1.5-7 % faster than 128-key tiles at 2 waves per SIMD.
// - d = 32: 8 waves, 128-key tiles (126 VGPRs, two workgroups per CU); taken
//   from 512 workgroups on.  2-5 % faster than the 4-wave shape.
template <int D, bool CAUSAL>
hipError_t launch_bf16_t(const LaunchArgs& a) {
  const int64_t items = (int64_t)(a.H_q / a.H_kv) * ((a.S + kRows - 1) / kRows);
  const int64_t wgs8 = a.B * a.H_kv * ((items + 7) / 8);
  if constexpr (D == 64) {
    if (wgs8 >= kCUs) return launch_bf16_w<D, CAUSAL, 8, 64>(a);
  } else {
    if (wgs8 >= 2 * kCUs) return launch_bf16_w<D, CAUSAL, 8, 128>(a);
  }
  return launch_bf16_w<D, CAUSAL, 4, 64>(a);
}

template <int D>
hipError_t launch_f32_t(const LaunchArgs& a) {
  const int64_t threads = a.B * a.S * a.H_q;
  const int64_t blocks = (threads + 255) / 256;
  // fp32 kernel keeps the sign of scale in c (no bf16 operand to negate)
  const float c = a.negate_q ? -a.c : a.c;
  hipLaunchKernelGGL((attn_fwd_f32<D>), dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.out, a.lse, a.B,
                     (int)a.S, a.H_q, a.H_kv, a.H_q / a.H_kv, c, a.causal);
  return hipGetLastError();
}

}  // namespace

int64_t bf16_grid_size(int64_t B, int64_t S, int32_t H_q, int32_t H_kv) {
  const int64_t R = H_q / H_kv;
  const int64_t items = R * ((S + kRows - 1) / kRows);
  return B * H_kv * ((items + 3) / 4);
}

hipError_t launch_attn_fwd(const LaunchArgs& a) {
  if (a.dtype == 0) {
    switch (a.d) {
      case 32: return a.causal ? launch_bf16_t<32, true>(a) : launch_bf16_t<32, false>(a);
      case 64: return a.causal ? launch_bf16_t<64, true>(a) : launch_bf16_t<64, false>(a);
      case 128: return a.causal ? launch_bf16_t<128, true>(a) : launch_bf16_t<128, false>(a);
    }
  } else {
    switch (a.d) {
      case 32: return launch_f32_t<32>(a);
      case 64: return launch_f32_t<64>(a);
      case 128: return launch_f32_t<128>(a);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace sqa
