/*
 * gen.c -- seeded synthetic inputs for the IBP workloads (GNN feature cache,
 * DLRM embedding table, LLM gradient buffer, integer id stream, a small fp32
 * gradient tensor, mixed id/dense feature rows) and their sample / gather index
 * sets.
 *
 * Holds no codec arithmetic: random numbers and value distributions only.  Both
 * the GPU path and the CPU oracle consume the bytes produced here.
 *
 * Random source: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used as a counter-based generator: draw i of
 * stream `key` is the SplitMix64 output function applied to key + (i+1)*gamma,
 * gamma = 0x9E3779B97F4A7C15.  Draws are independent of thread count and order.
 * Uniform doubles take the top 53 bits; normals use the Box-Muller transform
 * (cosine branch) on two uniform draws; fp32 values are the round-to-nearest-even
 * conversion of the double; bf16 values round the fp32 bits to nearest even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Independent stream key derived from a seed and a tag. */
uint64_t gen_key(uint64_t seed, uint64_t tag) { return mix64(seed * GAMMA + mix64(tag + 0x632BE59BD9B4E019ull)); }

uint64_t gen_u64(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

static double u01(uint64_t key, uint64_t i) { return (double)(gen_u64(key, i) >> 11) * 0x1.0p-53; }

static double normal(uint64_t key, uint64_t i) {
  const double u1 = 1.0 - u01(key, 2 * i); /* (0, 1] */
  const double u2 = u01(key, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return (uint16_t)((b >> 16) | 0x0040u); /* NaN */
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* out[i] = fp32(N(0,1) * sigma) */
void gen_normal_f32(uint64_t key, uint64_t n, double sigma, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = (float)(normal(key, (uint64_t)i) * sigma);
}

/* out[i] = max(z, +0.0) with z ~ N(0,1): half exact zeros, half |N(0,1)| */
void gen_relu_normal_f32(uint64_t key, uint64_t n, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    const double z = normal(key, (uint64_t)i);
    out[i] = z > 0.0 ? (float)z : 0.0f;
  }
}

/* Sparse features: out[i] = |N(0,1)| with probability p_nonzero, else +0.0. */
void gen_sparse_abs_normal_f32(uint64_t key, uint64_t n, double p_nonzero, float *out) {
  const uint64_t k_sel = gen_key(key, 1);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i)
    out[i] = u01(k_sel, (uint64_t)i) < p_nonzero ? (float)fabs(normal(key, (uint64_t)i)) : 0.0f;
}

/* out[i] = fp32(lo + (hi - lo) * U[0,1)) */
void gen_uniform_f32(uint64_t key, uint64_t n, double lo, double hi, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = (float)(lo + (hi - lo) * u01(key, (uint64_t)i));
}

/* bf16 gradient: N(0,1) * sigma, each element independently replaced with
 * probability p_out by an N(0,1) outlier. */
void gen_bf16_grad(uint64_t key, uint64_t n, double sigma, double p_out, uint16_t *out) {
  const uint64_t k_sel = gen_key(key, 1), k_out = gen_key(key, 2);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    const double z = u01(k_sel, (uint64_t)i) < p_out ? normal(k_out, (uint64_t)i) : normal(key, (uint64_t)i) * sigma;
    out[i] = f32_to_bf16_rne((float)z);
  }
}

/* Feature rows of a recommender's input: each row holds n_ids categorical ids
 * ~ U[0, 2^id_bits) as uint32, then n_dense dense features fp32(N(0,1)), all as
 * 32-bit words (a float's bits); 1 <= id_bits <= 32. */
void gen_feature_rows(uint64_t key, uint64_t nrows, unsigned n_ids, unsigned n_dense, unsigned id_bits,
                      uint32_t *out) {
  const uint64_t k_dense = gen_key(key, 1);
  const uint64_t row = (uint64_t)n_ids + n_dense;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)nrows; ++r) {
    uint32_t *o = out + (uint64_t)r * row;
    for (unsigned j = 0; j < n_ids; ++j)
      o[j] = (uint32_t)(gen_u64(key, (uint64_t)r * n_ids + j) >> (64 - id_bits));
    for (unsigned j = 0; j < n_dense; ++j) {
      const float f = (float)normal(k_dense, (uint64_t)r * n_dense + j);
      memcpy(&o[n_ids + j], &f, 4);
    }
  }
}

/* out[i] = U[0, 2^bits) as int64 */
void gen_ids(uint64_t key, uint64_t n, unsigned bits, int64_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = (int64_t)(gen_u64(key, (uint64_t)i) >> (64 - bits));
}

/* Each element independently (probability p) replaced by U[0, 2^bits). */
void gen_replace_ids(uint64_t key, uint64_t n, double p, unsigned bits, int64_t *out) {
  const uint64_t k_sel = gen_key(key, 1), k_val = gen_key(key, 2);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i)
    if (u01(k_sel, (uint64_t)i) < p) out[i] = (int64_t)(gen_u64(k_val, (uint64_t)i) >> (64 - bits));
}

/* k distinct row indices drawn uniformly from [0, nrows), ascending
 * (selection sampling, Knuth TAOCP vol. 2, Algorithm 3.4.2 S). */
int gen_sample_rows(uint64_t key, uint64_t nrows, uint64_t k, int64_t *out) {
  if (k > nrows) return 1;
  uint64_t m = 0;
  for (uint64_t t = 0; t < nrows && m < k; ++t)
    if ((double)(nrows - t) * u01(key, t) < (double)(k - m)) out[m++] = (int64_t)t;
  return m == k ? 0 : 2;
}

/* m ids uniform over [0, nrows) */
void gen_uniform_ids(uint64_t key, uint64_t nrows, uint64_t m, int64_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)m; ++j) out[j] = (int64_t)(u01(key, (uint64_t)j) * (double)nrows);
}

/* m ids from a bounded Zipf(s) over ranks 1..nrows (P(r) proportional to r^-s),
 * inverse CDF by binary search, rank r mapped to row perm[r-1] of a seeded
 * Fisher-Yates permutation of [0, nrows). */
int gen_zipf_ids(uint64_t key, uint64_t nrows, double s, uint64_t m, int64_t *out) {
  double *cdf = (double *)malloc(nrows * sizeof(double));
  int64_t *perm = (int64_t *)malloc(nrows * sizeof(int64_t));
  if (!cdf || !perm) {
    free(cdf);
    free(perm);
    return 1;
  }
  double acc = 0.0;
  for (uint64_t r = 0; r < nrows; ++r) {
    acc += pow((double)(r + 1), -s);
    cdf[r] = acc;
  }
  for (uint64_t r = 0; r < nrows; ++r) perm[r] = (int64_t)r;
  const uint64_t k_perm = gen_key(key, 7);
  for (uint64_t i = nrows - 1; i > 0; --i) {
    const uint64_t j = gen_u64(k_perm, i) % (i + 1);
    const int64_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
#pragma omp parallel for schedule(static)
  for (int64_t q = 0; q < (int64_t)m; ++q) {
    const double u = u01(key, (uint64_t)q) * acc;
    uint64_t lo = 0, hi = nrows - 1;
    while (lo < hi) {
      const uint64_t mid = (lo + hi) / 2;
      if (cdf[mid] > u) hi = mid; else lo = mid + 1;
    }
    out[q] = perm[lo];
  }
  free(cdf);
  free(perm);
  return 0;
}

/* out[j] = rows[ids[j]] for rows of row_bytes bytes (sample assembly). */
void gen_take_rows(const uint8_t *src, uint64_t row_bytes, const int64_t *ids, uint64_t m, uint8_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)m; ++j) memcpy(out + (uint64_t)j * row_bytes, src + (uint64_t)ids[j] * row_bytes, row_bytes);
}
