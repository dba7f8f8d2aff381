/*
 * Oracle for decoupled-head scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path never
 * calls it, and it shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes (plain definition, fp64, no blocking and no fusion):
 *
 *   - Sparse Query Attention (SQA abstract, "Sparse Query Attention (SQA): A
 *     Computationally Efficient Attention Mechanism with Query Heads
 *     Reduction"): the attention arithmetic is the ordinary one; SQA only
 *     changes how many query heads there are.  Query and key/value head
 *     counts are therefore independent arguments H_q and H_kv.
 *   - Head sharing ("Paper explainer: GQA - Grouped-Query Attention", section
 *     on the relation between MHA, MQA and GQA, the GQA equations and the
 *     grouping figure): the H_q query heads form H_kv groups of
 *     R = H_q / H_kv consecutive heads, and every head of group g reads K/V
 *     head g.  So query head h reads K/V head floor(h / R).  The same page's
 *     PyTorch module expands K/V with unsqueeze/expand/reshape, which puts
 *     K/V head g at query heads g*R ... g*R+R-1: the same map.
 *   - The attention itself (same page, PyTorch module, call to
 *     scaled_dot_product_attention with is_causal): per query row i,
 *     scores s_j = scale * <q_i, k_j>, weights softmax over j, output
 *     sum_j w_j v_j.  Written as on the quantum-attention review ("Beyond
 *     Classical Attention: Quantum Attention for Scalable Computation",
 *     proposed-method section): o = D(A)^-1 A V with A = exp(scores) and
 *     D the diagonal of row sums.
 *   - Causal: with equal query and key lengths, row i sees keys j <= i.
 *
 * Reading taken where the pages are silent: the row maximum is subtracted
 * before exponentiation (p_j = exp(s_j - m)).  In exact arithmetic this
 * leaves D(A)^-1 A V unchanged, because numerator and denominator are both
 * multiplied by exp(-m); it only keeps exp() from overflowing.
 *
 * Layout: all tensors dense BSHD, element (b, s, h, e) at ((b*S+s)*H+h)*d+e.
 * Input dtype code: 0 = bf16 (raw bits), 1 = fp32, 2 = fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 -> fp64: the bf16 bits are the upper half of an fp32; exact. */
static double load_elem(const void* p, int dtype, int64_t idx) {
  if (dtype == 0) {
    uint32_t u = (uint32_t)((const uint16_t*)p)[idx] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
  }
  if (dtype == 1) return (double)((const float*)p)[idx];
  return ((const double*)p)[idx];
}

/*
 * out: fp64, [B, n_out, H_q, d] where n_out = S if rows == NULL, else n_rows
 *      and output row r holds query position rows[r].
 * pairs_out (nullable): number of (b, h, i, j) score terms evaluated.
 * n_threads <= 0 uses the OpenMP default.
 * Returns 0 on success, -1 on invalid arguments, -2 if memory is short.
 */
int sqa_oracle_fwd(const void* q, const void* k, const void* v, int dtype, double* out,
                   int64_t B, int64_t S, int32_t H_q, int32_t H_kv, int32_t d, double scale,
                   int causal, const int64_t* rows, int64_t n_rows, int n_threads,
                   int64_t* pairs_out) {
  if (B < 0 || S < 0 || H_q < 1 || H_kv < 1 || d < 1) return -1;
  if (H_q % H_kv != 0) return -1;
  if (dtype < 0 || dtype > 2) return -1;
  if (causal != 0 && causal != 1) return -1;
  const int64_t n_out = rows ? n_rows : S;
  if (n_out < 0) return -1;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= S) return -1;
  if (pairs_out) *pairs_out = 0;
  const int64_t items = B * n_out * (int64_t)H_q;
  if (items == 0) return 0;

  const int32_t R = H_q / H_kv;
  int64_t pairs = 0;
  int failed = 0;
#ifdef _OPENMP
  if (n_threads <= 0) n_threads = omp_get_max_threads();
#else
  n_threads = 1;
#endif

#pragma omp parallel num_threads(n_threads) reduction(+ : pairs)
  {
    double* p = (double*)malloc((size_t)(S > 0 ? S : 1) * sizeof(double));
    double* acc = (double*)malloc((size_t)d * sizeof(double));
    if (!p || !acc) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < items; ++t) {
      if (!p || !acc) continue;
      const int64_t b = t / (n_out * H_q);
      const int64_t r = (t / H_q) % n_out;
      const int32_t h = (int32_t)(t % H_q);
      const int64_t i = rows ? rows[r] : r;
      const int32_t g = h / R; /* K/V head shared by query head h */
      const int64_t last = causal ? i : S - 1;
      const int64_t q_off = ((b * S + i) * H_q + h) * (int64_t)d;

      /* scores s_j = scale * <q_i, k_j> */
      double m = -INFINITY;
      for (int64_t j = 0; j <= last; ++j) {
        const int64_t k_off = ((b * S + j) * H_kv + g) * (int64_t)d;
        double dot = 0.0;
        for (int32_t e = 0; e < d; ++e) dot += load_elem(q, dtype, q_off + e) * load_elem(k, dtype, k_off + e);
        p[j] = scale * dot;
        if (p[j] > m) m = p[j];
      }
      /* A_ij = exp(s_j - m); D_ii = sum_j A_ij; o = D^-1 A V */
      double l = 0.0;
      for (int32_t e = 0; e < d; ++e) acc[e] = 0.0;
      for (int64_t j = 0; j <= last; ++j) {
        const double a = exp(p[j] - m);
        l += a;
        const int64_t v_off = ((b * S + j) * H_kv + g) * (int64_t)d;
        for (int32_t e = 0; e < d; ++e) acc[e] += a * load_elem(v, dtype, v_off + e);
      }
      double* o = out + ((b * n_out + r) * H_q + h) * (int64_t)d;
      for (int32_t e = 0; e < d; ++e) o[e] = acc[e] / l;
      pairs += last + 1;
    }
    free(p);
    free(acc);
  }
  if (failed) return -2;
  if (pairs_out) *pairs_out = pairs;
  return 0;
}

/*
 * Row log-normaliser of the same attention: lse[b, r, h] = log D_ii, where
 * D_ii = sum_j exp(s_j) is the row sum of A = exp(scores) in the D(A)^-1 A V
 * form (quantum-attention review, proposed-method section) and s_j =
 * scale * <q_i, k_j> over the visible keys j.  Computed as m + log(sum_j
 * exp(s_j - m)) with the row maximum m (exact in real arithmetic).  This is
 * the statistic a backward pass needs to rebuild the probabilities; the pages
 * do not name it, it is log of the normaliser they write.
 *
 * lse_out: fp64, [B, n_out, H_q] with n_out / rows as for sqa_oracle_fwd.
 */
int sqa_oracle_lse(const void* q, const void* k, int dtype, double* lse_out, int64_t B, int64_t S,
                   int32_t H_q, int32_t H_kv, int32_t d, double scale, int causal, const int64_t* rows,
                   int64_t n_rows, int n_threads) {
  if (B < 0 || S < 0 || H_q < 1 || H_kv < 1 || d < 1) return -1;
  if (H_q % H_kv != 0) return -1;
  if (dtype < 0 || dtype > 2) return -1;
  if (causal != 0 && causal != 1) return -1;
  const int64_t n_out = rows ? n_rows : S;
  if (n_out < 0) return -1;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= S) return -1;
  const int64_t items = B * n_out * (int64_t)H_q;
  if (items == 0) return 0;
  const int32_t R = H_q / H_kv;
  int failed = 0;
#ifdef _OPENMP
  if (n_threads <= 0) n_threads = omp_get_max_threads();
#else
  n_threads = 1;
#endif
#pragma omp parallel num_threads(n_threads)
  {
    double* p = (double*)malloc((size_t)(S > 0 ? S : 1) * sizeof(double));
    if (!p) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < items; ++t) {
      if (!p) continue;
      const int64_t b = t / (n_out * H_q);
      const int64_t r = (t / H_q) % n_out;
      const int32_t h = (int32_t)(t % H_q);
      const int64_t i = rows ? rows[r] : r;
      const int32_t g = h / R;
      const int64_t last = causal ? i : S - 1;
      const int64_t q_off = ((b * S + i) * H_q + h) * (int64_t)d;
      double m = -INFINITY;
      for (int64_t j = 0; j <= last; ++j) {
        const int64_t k_off = ((b * S + j) * H_kv + g) * (int64_t)d;
        double dot = 0.0;
        for (int32_t e = 0; e < d; ++e) dot += load_elem(q, dtype, q_off + e) * load_elem(k, dtype, k_off + e);
        p[j] = scale * dot;
        if (p[j] > m) m = p[j];
      }
      double l = 0.0;
      for (int64_t j = 0; j <= last; ++j) l += exp(p[j] - m);
      lse_out[(b * n_out + r) * H_q + h] = m + log(l);
    }
    free(p);
  }
  return failed ? -2 : 0;
}

/*
 * Gradient of the same attention with respect to q, k and v, for an upstream
 * gradient dout = dL/dout.  The pages define only the forward computation;
 * this is its exact derivative, written out in fp64:
 *
 *   p_ij  = exp(s_ij - lse_i)           s_ij = scale * <q_i, k_j>, j visible
 *   dp_ij = <dout_i, v_j>
 *   D_i   = sum_j p_ij dp_ij            (= <dout_i, out_i>)
 *   ds_ij = p_ij (dp_ij - D_i)          (softmax Jacobian)
 *   dq_i  = scale * sum_j ds_ij k_j
 *   dk_j  = scale * sum over query heads h of group g, rows i: ds_ij q_i
 *   dv_j  =         sum over query heads h of group g, rows i: p_ij dout_i
 *
 * Key/value heads are shared by the R query heads of their group (GQA
 * explainer: grouping figure and the expand in the PyTorch module), so their
 * gradients sum over those heads.  Pass 1 runs per query row (lse_i, D_i,
 * dq_i); pass 2 per key (dk_j, dv_j), reusing lse_i and D_i.
 * Outputs are fp64 in BSHD layout: dq [B,S,H_q,d], dk and dv [B,S,H_kv,d].
 */
int sqa_oracle_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype, double* dq,
                   double* dk, double* dv, int64_t B, int64_t S, int32_t H_q, int32_t H_kv, int32_t d,
                   double scale, int causal, int n_threads) {
  if (B < 0 || S < 0 || H_q < 1 || H_kv < 1 || d < 1) return -1;
  if (H_q % H_kv != 0) return -1;
  if (dtype < 0 || dtype > 2) return -1;
  if (causal != 0 && causal != 1) return -1;
  const int64_t rows_q = B * S * (int64_t)H_q;
  if (rows_q == 0) return 0;
  const int32_t R = H_q / H_kv;
  double* lse = (double*)malloc((size_t)rows_q * sizeof(double));
  double* Dd = (double*)malloc((size_t)rows_q * sizeof(double));
  if (!lse || !Dd) {
    free(lse);
    free(Dd);
    return -2;
  }
  int failed = 0;
#ifdef _OPENMP
  if (n_threads <= 0) n_threads = omp_get_max_threads();
#else
  n_threads = 1;
#endif

  /* pass 1: per (b, i, h) row */
#pragma omp parallel num_threads(n_threads)
  {
    double* s = (double*)malloc((size_t)S * sizeof(double));
    double* dp = (double*)malloc((size_t)S * sizeof(double));
    if (!s || !dp) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < rows_q; ++t) {
      if (!s || !dp) continue;
      const int64_t b = t / ((int64_t)S * H_q);
      const int64_t i = (t / H_q) % S;
      const int32_t h = (int32_t)(t % H_q);
      const int32_t g = h / R;
      const int64_t last = causal ? i : S - 1;
      const int64_t qo = ((b * S + i) * H_q + h) * (int64_t)d;
      double m = -INFINITY;
      for (int64_t j = 0; j <= last; ++j) {
        const int64_t ko = ((b * S + j) * H_kv + g) * (int64_t)d;
        double dot = 0.0, dd = 0.0;
        for (int32_t e = 0; e < d; ++e) {
          dot += load_elem(q, dtype, qo + e) * load_elem(k, dtype, ko + e);
          dd += load_elem(dout, dtype, qo + e) * load_elem(v, dtype, ko + e);
        }
        s[j] = scale * dot;
        dp[j] = dd;
        if (s[j] > m) m = s[j];
      }
      double l = 0.0;
      for (int64_t j = 0; j <= last; ++j) l += exp(s[j] - m);
      const double L = m + log(l);
      double Di = 0.0;
      for (int64_t j = 0; j <= last; ++j) Di += exp(s[j] - L) * dp[j];
      lse[t] = L;
      Dd[t] = Di;
      double* dqi = dq + qo;
      for (int32_t e = 0; e < d; ++e) dqi[e] = 0.0;
      for (int64_t j = 0; j <= last; ++j) {
        const double ds = exp(s[j] - L) * (dp[j] - Di);
        const int64_t ko = ((b * S + j) * H_kv + g) * (int64_t)d;
        for (int32_t e = 0; e < d; ++e) dqi[e] += ds * load_elem(k, dtype, ko + e);
      }
      for (int32_t e = 0; e < d; ++e) dqi[e] *= scale;
    }
    free(s);
    free(dp);
  }
  if (failed) {
    free(lse);
    free(Dd);
    return -2;
  }

  /* pass 2: per (b, j, g) key */
  const int64_t rows_k = B * S * (int64_t)H_kv;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
  for (int64_t t = 0; t < rows_k; ++t) {
    const int64_t b = t / ((int64_t)S * H_kv);
    const int64_t j = (t / H_kv) % S;
    const int32_t g = (int32_t)(t % H_kv);
    const int64_t ko = ((b * S + j) * H_kv + g) * (int64_t)d;
    double* dkj = dk + ko;
    double* dvj = dv + ko;
    for (int32_t e = 0; e < d; ++e) dkj[e] = dvj[e] = 0.0;
    for (int32_t h = g * R; h < (g + 1) * R; ++h)
      for (int64_t i = causal ? j : 0; i < S; ++i) {
        const int64_t qo = ((b * S + i) * H_q + h) * (int64_t)d;
        const int64_t row = (b * S + i) * H_q + h;
        double dot = 0.0, dd = 0.0;
        for (int32_t e = 0; e < d; ++e) {
          dot += load_elem(q, dtype, qo + e) * load_elem(k, dtype, ko + e);
          dd += load_elem(dout, dtype, qo + e) * load_elem(v, dtype, ko + e);
        }
        const double p = exp(scale * dot - lse[row]);
        const double ds = p * (dd - Dd[row]);
        for (int32_t e = 0; e < d; ++e) {
          dvj[e] += p * load_elem(dout, dtype, qo + e);
          dkj[e] += ds * load_elem(q, dtype, qo + e);
        }
      }
    for (int32_t e = 0; e < d; ++e) dkj[e] *= scale;
  }
  free(lse);
  free(Dd);
  return 0;
}

/*
 * dq rows only (pass 1 of sqa_oracle_bwd restricted to the query positions
 * `rows`, all batches and heads): dq_out is fp64 [B, n_rows, H_q, d].  Each
 * row needs only its own keys, so a sample of rows costs a sample of the work.
 */
int sqa_oracle_bwd_dq_rows(const void* q, const void* k, const void* v, const void* dout, int dtype, double* dq_out,
                           int64_t B, int64_t S, int32_t H_q, int32_t H_kv, int32_t d, double scale, int causal,
                           const int64_t* rows, int64_t n_rows, int n_threads) {
  if (B < 0 || S < 0 || H_q < 1 || H_kv < 1 || d < 1 || H_q % H_kv != 0) return -1;
  if (dtype < 0 || dtype > 2 || (causal != 0 && causal != 1) || !rows || n_rows < 0) return -1;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= S) return -1;
  const int64_t items = B * n_rows * (int64_t)H_q;
  if (items == 0) return 0;
  const int32_t R = H_q / H_kv;
  int failed = 0;
#ifdef _OPENMP
  if (n_threads <= 0) n_threads = omp_get_max_threads();
#else
  n_threads = 1;
#endif
#pragma omp parallel num_threads(n_threads)
  {
    double* s = (double*)malloc((size_t)S * sizeof(double));
    double* dp = (double*)malloc((size_t)S * sizeof(double));
    if (!s || !dp) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < items; ++t) {
      if (!s || !dp) continue;
      const int64_t b = t / (n_rows * H_q);
      const int64_t r = (t / H_q) % n_rows;
      const int32_t h = (int32_t)(t % H_q);
      const int64_t i = rows[r];
      const int32_t g = h / R;
      const int64_t last = causal ? i : S - 1;
      const int64_t qo = ((b * S + i) * H_q + h) * (int64_t)d;
      double m = -INFINITY;
      for (int64_t j = 0; j <= last; ++j) {
        const int64_t ko = ((b * S + j) * H_kv + g) * (int64_t)d;
        double dot = 0.0, dd = 0.0;
        for (int32_t e = 0; e < d; ++e) {
          dot += load_elem(q, dtype, qo + e) * load_elem(k, dtype, ko + e);
          dd += load_elem(dout, dtype, qo + e) * load_elem(v, dtype, ko + e);
        }
        s[j] = scale * dot;
        dp[j] = dd;
        if (s[j] > m) m = s[j];
      }
      double l = 0.0;
      for (int64_t j = 0; j <= last; ++j) l += exp(s[j] - m);
      const double L = m + log(l);
      double Di = 0.0;
      for (int64_t j = 0; j <= last; ++j) Di += exp(s[j] - L) * dp[j];
      double* o = dq_out + ((b * n_rows + r) * H_q + h) * (int64_t)d;
      for (int32_t e = 0; e < d; ++e) o[e] = 0.0;
      for (int64_t j = 0; j <= last; ++j) {
        const double ds = exp(s[j] - L) * (dp[j] - Di);
        const int64_t ko = ((b * S + j) * H_kv + g) * (int64_t)d;
        for (int32_t e = 0; e < d; ++e) o[e] += ds * load_elem(k, dtype, ko + e);
      }
      for (int32_t e = 0; e < d; ++e) o[e] *= scale;
    }
    free(s);
    free(dp);
  }
  return failed ? -2 : 0;
}

/*
 * Decode: one new query token per sequence against that sequence's
 * key/value cache.  The GQA explainer's background section puts the cache
 * at the centre of inference cost (2*G*d_h values stored per token, read in
 * full for every generated token); the SQA abstract contrasts this
 * bandwidth-bound regime with its compute-bound one.  The result is the
 * ordinary attention of a single query row:
 *
 *   q    [B, H_q, d]          the token's query heads
 *   k, v [B, S_max, H_kv, d]  the cache, BSHD, positions 0 .. len_b-1 valid
 *   seqlens[b]                valid cache length of sequence b (host array;
 *                             NULL = S_max for every sequence)
 *   out  [B, H_q, d] fp64,  lse [B, H_q] fp64 (nullable)
 *
 *   o[b,h] = sum_{j < len_b} softmax_j(scale * <q[b,h], k[b,j,g]>) v[b,j,g],
 *   lse[b,h] = log sum_{j < len_b} exp(scale * <q[b,h], k[b,j,g]>),
 *   g = floor(h / R) as in the forward.
 *
 * This is the causal forward's row len_b - 1 when the token sits at that
 * position (it sees every cached key up to and including its own).
 * Readings where the pages say nothing: len_b > S_max is taken as S_max; an
 * empty cache (len_b <= 0) gives the empty sum: o = 0 and lse = -inf.
 */
int sqa_oracle_decode(const void* q, const void* k, const void* v, int dtype, const int64_t* seqlens, double* out,
                      double* lse_out, int64_t B, int64_t S_max, int32_t H_q, int32_t H_kv, int32_t d, double scale,
                      int n_threads) {
  if (B < 0 || S_max < 0 || H_q < 1 || H_kv < 1 || d < 1 || H_q % H_kv != 0) return -1;
  if (dtype < 0 || dtype > 2) return -1;
  const int64_t items = B * (int64_t)H_q;
  if (items == 0) return 0;
  const int32_t R = H_q / H_kv;
  int failed = 0;
#ifdef _OPENMP
  if (n_threads <= 0) n_threads = omp_get_max_threads();
#else
  n_threads = 1;
#endif
#pragma omp parallel num_threads(n_threads)
  {
    double* p = (double*)malloc((size_t)(S_max > 0 ? S_max : 1) * sizeof(double));
    double* acc = (double*)malloc((size_t)d * sizeof(double));
    if (!p || !acc) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < items; ++t) {
      if (!p || !acc) continue;
      const int64_t b = t / H_q;
      const int32_t h = (int32_t)(t % H_q);
      const int32_t g = h / R;
      int64_t len = seqlens ? seqlens[b] : S_max;
      if (len > S_max) len = S_max;
      double* o = out + t * (int64_t)d;
      if (len <= 0) {
        for (int32_t e = 0; e < d; ++e) o[e] = 0.0;
        if (lse_out) lse_out[t] = -INFINITY;
        continue;
      }
      const int64_t q_off = t * (int64_t)d;
      double m = -INFINITY;
      for (int64_t j = 0; j < len; ++j) {
        const int64_t k_off = ((b * S_max + j) * H_kv + g) * (int64_t)d;
        double dot = 0.0;
        for (int32_t e = 0; e < d; ++e) dot += load_elem(q, dtype, q_off + e) * load_elem(k, dtype, k_off + e);
        p[j] = scale * dot;
        if (p[j] > m) m = p[j];
      }
      double l = 0.0;
      for (int32_t e = 0; e < d; ++e) acc[e] = 0.0;
      for (int64_t j = 0; j < len; ++j) {
        const double a = exp(p[j] - m);
        l += a;
        const int64_t v_off = ((b * S_max + j) * H_kv + g) * (int64_t)d;
        for (int32_t e = 0; e < d; ++e) acc[e] += a * load_elem(v, dtype, v_off + e);
      }
      for (int32_t e = 0; e < d; ++e) o[e] = acc[e] / l;
      if (lse_out) lse_out[t] = m + log(l);
    }
    free(p);
    free(acc);
  }
  return failed ? -2 : 0;
}
