/*
 * Seeded synthetic inputs for decoupled-head attention (shared by the oracle
 * side and the GPU side of every comparison).
 *
 * This file holds random-number generation and number-format encoding only:
 * none of the attention arithmetic lives here.
 *
 *   counter hash  h(seed, stream, c) = mix(mix(seed ^ stream*0xD1B54A32D192ED03) ^ c)
 *                 where mix() is the SplitMix64 output step (Steele, Lea and
 *                 Flood, "Fast splittable pseudorandom number generators",
 *                 OOPSLA 2014): add the golden gamma, then two xor-shift-multiply
 *                 rounds and a final xor-shift.
 *   uniform       u(c) = ((h >> 11) + 1) * 2^-53, in (0, 1]
 *   normal        z(i) = sqrt(-2 ln u(2i)) * cos(2 pi u(2i+1))   (Box-Muller)
 *   encodings     fp64 -> fp32 by C conversion (round to nearest even),
 *                 fp32 -> bf16 by round-to-nearest-even on the upper 16 bits.
 *
 * Every value depends only on (seed, stream, flat element index), never on
 * the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t ctr_hash(uint64_t key, uint64_t c) { return mix64(key ^ c); }

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed ^ (stream * 0xD1B54A32D192ED03ull));
}

static inline double uniform01(uint64_t key, uint64_t c) {
  return (double)((ctr_hash(key, c) >> 11) + 1) * 0x1.0p-53;
}

static inline double normal_at(uint64_t key, int64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = uniform01(key, 2 * (uint64_t)i);
  double u2 = uniform01(key, 2 * (uint64_t)i + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint64_t sqa_gen_splitmix64(uint64_t state) { return mix64(state); }

uint64_t sqa_gen_hash(uint64_t seed, uint64_t stream, uint64_t c) { return ctr_hash(stream_key(seed, stream), c); }

double sqa_gen_uniform(uint64_t seed, uint64_t stream, uint64_t c) { return uniform01(stream_key(seed, stream), c); }

/* out[i] = (float)(mul * z(i)), i < n */
void sqa_gen_normal_f32(uint64_t seed, uint64_t stream, double mul, int64_t n, float* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(mul * normal_at(key, i));
}

/* out[i] = bf16_rne((float)(mul * z(i))), stored as raw bf16 bits */
void sqa_gen_normal_bf16(uint64_t seed, uint64_t stream, double mul, int64_t n, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)(mul * normal_at(key, i)));
}

/* fp32 -> bf16 (round to nearest even) for n values */
void sqa_gen_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

/* Choose n distinct positions in [0, S) by a seeded partial Fisher-Yates
 * shuffle (draw j uses counter j), returned in ascending order.
 * Returns 0, or -1 if n > S or memory is short. */
int sqa_gen_select_positions(uint64_t seed, uint64_t stream, int64_t S, int64_t n, int64_t* out) {
  if (n < 0 || n > S) return -1;
  int64_t* perm = (int64_t*)malloc((size_t)(S > 0 ? S : 1) * sizeof(int64_t));
  if (!perm) return -1;
  for (int64_t i = 0; i < S; ++i) perm[i] = i;
  uint64_t key = stream_key(seed, stream);
  for (int64_t j = 0; j < n; ++j) {
    uint64_t range = (uint64_t)(S - j);
    uint64_t r = (uint64_t)(((unsigned __int128)ctr_hash(key, (uint64_t)j) * range) >> 64);
    int64_t t = perm[j];
    perm[j] = perm[j + (int64_t)r];
    perm[j + (int64_t)r] = t;
  }
  /* ascending order: counting sort over a byte mask */
  unsigned char* mark = (unsigned char*)calloc((size_t)(S > 0 ? S : 1), 1);
  if (!mark) { free(perm); return -1; }
  for (int64_t j = 0; j < n; ++j) mark[perm[j]] = 1;
  int64_t c = 0;
  for (int64_t i = 0; i < S; ++i) if (mark[i]) out[c++] = i;
  free(mark);
  free(perm);
  return 0;
}

/* x is [B, S, row_elems] bf16 bits; multiply the rows at the n given
 * positions (every b) by factor, re-encoding with round-to-nearest-even. */
void sqa_gen_scale_positions_bf16(uint16_t* x, int64_t B, int64_t S, int64_t row_elems,
                                  const int64_t* pos, int64_t n, float factor) {
  for (int64_t b = 0; b < B; ++b)
    for (int64_t j = 0; j < n; ++j) {
      uint16_t* row = x + (b * S + pos[j]) * row_elems;
      for (int64_t e = 0; e < row_elems; ++e) row[e] = f32_to_bf16_rne(bf16_to_f32(row[e]) * factor);
    }
}
