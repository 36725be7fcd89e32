/*
 * Seeded synthetic inputs for the sparse-attention KV slot buffer:
 * bf16 K/V rows, bf16 queries and per-step top-k selections.
 *
 * This file holds no part of the buffer-management method itself (no
 * matching, no eviction, no attention).  Both the HIP path and the CPU
 * oracle consume what it writes, so they see identical inputs.
 *
 * Generator definition (all integer arithmetic is exact and portable):
 *   mix(x)        the splitmix64 finaliser (Steele, Lea, Flood, "Fast
 *                 splittable pseudorandom number generators", 2014).
 *   rnd(key, i) = mix(key + (i + 1) * 0x9E3779B97F4A7C15)   -- the i-th
 *                 output of a splitmix64 stream started at `key`, so any
 *                 element can be drawn without drawing the ones before it.
 *   key derivation: key(a, b, ...) = mix(mix(mix(seed ^ a) ^ b) ^ ...).
 *   unit01(x)   = (x >> 11) * 2^-53  in [0, 1).
 *   normal pairs: Box-Muller on (unit01(rnd(k, 2p)), unit01(rnd(k, 2p+1))),
 *                 z0 = sqrt(-2 ln(1-a)) cos(2 pi b), z1 = ... sin(2 pi b),
 *                 evaluated in double, rounded to float, then to bf16 with
 *                 round-to-nearest-even.
 *   bounded(x, n) = floor(x * n / 2^64) (Lemire's multiply-shift).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix(uint64_t x) {
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ULL;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBULL;
  return x ^ (x >> 31);
}
static inline uint64_t rnd(uint64_t key, uint64_t i) { return mix(key + (i + 1) * GOLDEN); }
static inline double unit01(uint64_t x) { return (double)(x >> 11) * (1.0 / 9007199254740992.0); }
static inline uint64_t bounded(uint64_t x, uint64_t n) {
  return (uint64_t)(((unsigned __int128)x * n) >> 64);
}

/* purposes: separate streams for K/V, queries, permutations, selections */
enum { P_KV = 1, P_Q = 2, P_PERM = 3, P_SEL = 4 };

uint64_t tg_key2(uint64_t seed, uint64_t a, uint64_t b) { return mix(mix(seed ^ a) ^ b); }
uint64_t tg_key3(uint64_t seed, uint64_t a, uint64_t b, uint64_t c) {
  return mix(mix(mix(seed ^ a) ^ b) ^ c);
}
uint64_t tg_rnd(uint64_t key, uint64_t i) { return rnd(key, i); }

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)(u >> 16); /* inf/nan: not produced */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Fill n bf16 values with N(0,1) draws from stream `key`; element e of the
 * stream is element (first + e).  `first` must be even. */
static void fill_normal_bf16(uint64_t key, uint64_t first, uint64_t n, uint16_t* out) {
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t p0 = first / 2, np = (n + 1) / 2;
#pragma omp parallel for schedule(static)
  for (int64_t pp = 0; pp < (int64_t)np; ++pp) {
    uint64_t p = p0 + (uint64_t)pp;
    double a = unit01(rnd(key, 2 * p)), b = unit01(rnd(key, 2 * p + 1));
    double r = sqrt(-2.0 * log(1.0 - a));
    double z0 = r * cos(two_pi * b), z1 = r * sin(two_pi * b);
    uint64_t e = 2 * (uint64_t)pp;
    out[e] = f32_to_bf16_rne((float)z0);
    if (e + 1 < n) out[e + 1] = f32_to_bf16_rne((float)z1);
  }
}

/* K/V rows of one unit: n_entries rows of row_elems bf16, drawn from the
 * (seed, P_KV, unit) stream in row-major order.  Rows [row0, row0+nrows)
 * are written to out. */
void tg_fill_kv_rows(uint64_t seed, int64_t unit, int64_t row_elems, int64_t row0, int64_t nrows,
                     uint16_t* out) {
  uint64_t key = tg_key2(seed, P_KV, (uint64_t)unit);
  uint64_t first = (uint64_t)row0 * (uint64_t)row_elems;
  uint64_t n = (uint64_t)nrows * (uint64_t)row_elems;
  if (first & 1) { /* keep pairs aligned: draw one extra leading value */
    uint16_t* tmp = (uint16_t*)malloc((n + 1) * 2);
    fill_normal_bf16(key, first - 1, n + 1, tmp);
    memcpy(out, tmp + 1, n * 2);
    free(tmp);
  } else {
    fill_normal_bf16(key, first, n, out);
  }
}

/* Whole host KV: units x n_entries x row_elems, unit-major. */
void tg_fill_kv(uint64_t seed, int64_t units, int64_t n_entries, int64_t row_elems, uint16_t* out) {
  for (int64_t u = 0; u < units; ++u)
    tg_fill_kv_rows(seed, u, row_elems, 0, n_entries, out + u * n_entries * row_elems);
}

/* Queries of decode step `step`: n bf16 values from the (seed, P_Q, step) stream. */
void tg_fill_q(uint64_t seed, int64_t step, int64_t n, uint16_t* out) {
  fill_normal_bf16(tg_key2(seed, P_Q, (uint64_t)step), 0, (uint64_t)n, out);
}

/* ---------------------------------------------------------------- selections */

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Zipf(s) CDF over ranks 1..n: cdf[r-1] = sum_{i<=r} i^-s / H. */
static double* zipf_cdf(int64_t n, double s) {
  double* c = (double*)malloc(sizeof(double) * (size_t)n);
  double acc = 0.0;
  for (int64_t r = 1; r <= n; ++r) { acc += pow((double)r, -s); c[r - 1] = acc; }
  for (int64_t r = 0; r < n; ++r) c[r] /= acc;
  c[n - 1] = 1.0;
  return c;
}
/* smallest rank index r (0-based) with cdf[r] > x */
static int64_t zipf_rank(const double* cdf, int64_t n, double x) {
  int64_t lo = 0, hi = n - 1;
  while (lo < hi) {
    int64_t mid = (lo + hi) / 2;
    if (cdf[mid] > x) hi = mid; else lo = mid + 1;
  }
  return lo;
}

/* Fisher-Yates permutation of 0..n-1 from the (seed, P_PERM, unit) stream. */
void tg_permutation(uint64_t seed, int64_t unit, int64_t n, int32_t* perm) {
  uint64_t key = tg_key2(seed, P_PERM, (uint64_t)unit);
  for (int64_t i = 0; i < n; ++i) perm[i] = (int32_t)i;
  uint64_t c = 0;
  for (int64_t i = n - 1; i >= 1; --i) {
    int64_t j = (int64_t)bounded(rnd(key, c++), (uint64_t)(i + 1));
    int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
  }
}

typedef struct { uint64_t key, ctr; } stream_t;
static inline uint64_t next(stream_t* s) { return rnd(s->key, s->ctr++); }

/* Keep `keep` entries of prev (size k) chosen uniformly without replacement
 * (partial Fisher-Yates on a copy), then add draws from the Zipf tail that
 * are not in `excl` and not already taken, until `k_out` entries.  mark[] is a
 * scratch array of n bytes, all zero on entry and on exit. */
static void draw_overlapping(stream_t* st, const int32_t* prev, int64_t k_prev, int64_t keep,
                             const uint8_t* excl_mark, const double* cdf, const int32_t* perm,
                             int64_t n, int64_t k_out, uint8_t* mark, int32_t* out, int32_t* tmp) {
  memcpy(tmp, prev, sizeof(int32_t) * (size_t)k_prev);
  for (int64_t i = 0; i < keep; ++i) {
    int64_t j = i + (int64_t)bounded(next(st), (uint64_t)(k_prev - i));
    int32_t t = tmp[i]; tmp[i] = tmp[j]; tmp[j] = t;
    out[i] = tmp[i];
    mark[tmp[i]] = 1;
  }
  int64_t got = keep;
  while (got < k_out) {
    int32_t pos = perm[zipf_rank(cdf, n, unit01(next(st)))];
    if (mark[pos] || (excl_mark && excl_mark[pos])) continue;
    mark[pos] = 1;
    out[got++] = pos;
  }
  for (int64_t i = 0; i < k_out; ++i) mark[out[i]] = 0;
  qsort(out, (size_t)k_out, sizeof(int32_t), cmp_i32);
}

/*
 * Selections for `steps` decode steps of `units` units, T query tokens each:
 * out[step][unit][T][k] int32, every list strictly ascending in [0, n).
 *   mode 0 (natural): step 0 draws k distinct Zipf(zipf_s) positions over a
 *     per-unit random permutation; step t keeps round(f*k) entries of token
 *     0's previous list, uniformly, and fills up with Zipf draws outside the
 *     previous list, so consecutive lists overlap in exactly round(f*k).
 *     Token j >= 1 keeps round(f_shared*k) entries of token 0's list of the
 *     same step and fills up with Zipf draws outside it.
 *   mode 1 (all-hit): every step repeats step 0.
 *   mode 2 (all-miss): token j of step t is window w = (t*T + j) mod (n/k) of
 *     the permutation, sorted; windows are disjoint.
 *   mode 3 (skewed): units u with u % 8 == 0 follow mode 2, all other units
 *     follow mode 1, so a few units carry every transfer of a step.
 * Returns 0, or -1 if the arguments cannot be satisfied.
 */
int tg_selections(uint64_t seed, int64_t units, int64_t n, int64_t k, int64_t T, int64_t steps,
                  double f, double f_shared, double zipf_s, int mode, int32_t* out) {
  if (k <= 0 || k * 2 > n || T < 1 || steps < 1) return -1;
  if ((mode == 2 || mode == 3) && (n / k) < 1) return -1;
  double* cdf = zipf_cdf(n, zipf_s);
  int64_t keep = (int64_t)floor(f * (double)k + 0.5);
  int64_t keep_sh = (int64_t)floor(f_shared * (double)k + 0.5);
  if (keep > k) keep = k;
  if (keep_sh > k) keep_sh = k;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    uint8_t* mark = (uint8_t*)calloc((size_t)n, 1);
    uint8_t* excl = (uint8_t*)calloc((size_t)n, 1);
    int32_t* tmp = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    tg_permutation(seed, u, n, perm);
    const size_t tk = (size_t)(T * k);
    for (int64_t t = 0; t < steps; ++t) {
      stream_t st = {tg_key3(seed, P_SEL, (uint64_t)u, (uint64_t)t), 0};
      int32_t* cur = out + ((size_t)t * (size_t)units + (size_t)u) * tk;
      const int umode = mode == 3 ? (u % 8 == 0 ? 2 : 1) : mode;
      if (umode == 2) {
        for (int64_t j = 0; j < T; ++j) {
          int64_t w = (t * T + j) % (n / k);
          memcpy(cur + j * k, perm + w * k, sizeof(int32_t) * (size_t)k);
          qsort(cur + j * k, (size_t)k, sizeof(int32_t), cmp_i32);
        }
        continue;
      }
      if (t == 0 || umode == 1) {
        if (t > 0) { memcpy(cur, cur - (size_t)units * tk, sizeof(int32_t) * tk); continue; }
        draw_overlapping(&st, NULL, 0, 0, NULL, cdf, perm, n, k, mark, cur, tmp);
      } else {
        const int32_t* prev = cur - (size_t)units * tk; /* token 0 of step t-1 */
        for (int64_t i = 0; i < k; ++i) excl[prev[i]] = 1;
        draw_overlapping(&st, prev, k, keep, excl, cdf, perm, n, k, mark, cur, tmp);
        for (int64_t i = 0; i < k; ++i) excl[prev[i]] = 0;
      }
      for (int64_t j = 1; j < T; ++j) {
        for (int64_t i = 0; i < k; ++i) excl[cur[i]] = 1;
        draw_overlapping(&st, cur, k, keep_sh, excl, cdf, perm, n, k, mark, cur + j * k, tmp);
        for (int64_t i = 0; i < k; ++i) excl[cur[i]] = 0;
      }
    }
    free(perm); free(mark); free(excl); free(tmp);
  }
  free(cdf);
  return bad ? -1 : 0;
}
