/*
 * e-means CPU oracle: the direct-definition loops.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain checker that the GPU
 * library is compared against. Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load it; the library never does.
 *
 * Everything here is written from the definitions, in fp64, with no blocking,
 * tiling or algebraic rewriting:
 *   - squared Euclidean distance  sum_t (x_t - c_t)^2  and its argmin
 *     (k-means objective, blog "k-means Reads Your Data 25 Times", section on
 *     Lloyd's 1957 algorithm, MSE formula);
 *   - per-cluster count n_j and sum s_j of a batch (faiss e_means README,
 *     "How the centroid updates work");
 *   - Philox4x64-10, the counter-based generator of Salmon, Moraes, Dror and
 *     Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11);
 *   - a keyed bijection on [0, n): a 4-round balanced Feistel network
 *     (Luby-Rackoff) whose round function is Philox, restricted to [0, n) by
 *     cycle-walking (Black and Rogaway, "Ciphers with Arbitrary Finite
 *     Domains", 2002). It stands for the "fresh random order every pass" of
 *     the README's batch loop ("Data too big for memory").
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC -o libemeans_ref.so emeans_ref.c
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Philox4x64-10 (Salmon et al. 2011): multipliers, Weyl key increments and */
/* the round S-box as published.                                            */
/* ------------------------------------------------------------------------ */
static const uint64_t PH_M0 = 0xD2E7470EE14C6C93ULL;
static const uint64_t PH_M1 = 0xCA5A826395121157ULL;
static const uint64_t PH_W0 = 0x9E3779B97F4A7C15ULL;
static const uint64_t PH_W1 = 0xBB67AE8584CAA73BULL;

void ref_philox4x64(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
  uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint64_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += PH_W0;
      k1 += PH_W1;
    }
    unsigned __int128 p0 = (unsigned __int128)PH_M0 * c0;
    unsigned __int128 p1 = (unsigned __int128)PH_M1 * c2;
    uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
    uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    uint64_t n0 = hi1 ^ c1 ^ k0;
    uint64_t n1 = lo1;
    uint64_t n2 = hi0 ^ c3 ^ k1;
    uint64_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* ------------------------------------------------------------------------ */
/* Keyed permutation of [0, n).                                              */
/*   half width h = max(1, ceil(bits(n-1) / 2)), domain 2^(2h) >= n          */
/*   round r (0..3): F = Philox(ctr=(R, r, pass, stream), key=(seed, 0))[0]  */
/*                   (L, R) <- (R, L xor (F mod 2^h))                        */
/*   cycle-walk: re-encrypt while the value is >= n.                         */
/* ------------------------------------------------------------------------ */
static int ref_half_bits(uint64_t n) {
  int m = 0;
  while (m < 64 && (n - 1) >> m) ++m; /* bits needed for n-1 (0 when n == 1) */
  int h = (m + 1) / 2;
  return h < 1 ? 1 : h;
}

static uint64_t ref_feistel(uint64_t v, int h, uint64_t seed, uint64_t stream, uint64_t pass) {
  const uint64_t mask = (h >= 64) ? ~0ULL : ((1ULL << h) - 1);
  uint64_t L = v >> h, R = v & mask;
  for (uint64_t r = 0; r < 4; ++r) {
    uint64_t ctr[4] = {R, r, pass, stream};
    uint64_t key[2] = {seed, 0};
    uint64_t o[4];
    ref_philox4x64(ctr, key, o);
    uint64_t nl = R;
    uint64_t nr = L ^ (o[0] & mask);
    L = nl;
    R = nr;
  }
  return (L << h) | R;
}

int64_t ref_perm_at(uint64_t n, uint64_t seed, uint64_t stream, uint64_t pass, uint64_t i) {
  int h = ref_half_bits(n);
  uint64_t v = ref_feistel(i, h, seed, stream, pass);
  while (v >= n) v = ref_feistel(v, h, seed, stream, pass);
  return (int64_t)v;
}

void ref_perm_range(uint64_t n, uint64_t seed, uint64_t stream, uint64_t pass, uint64_t start,
                    uint64_t count, int64_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)count; ++i) out[i] = ref_perm_at(n, seed, stream, pass, start + (uint64_t)i);
}

/* ------------------------------------------------------------------------ */
/* Element access: dtype 0 = fp32, 1 = bf16 (stored as the high 16 bits of  */
/* an fp32), 2 = int8 codes, 4 = IEEE fp16, 5 = uint8 values, 3 = FP8 E4M3  */
/* codes (OCP: sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent */
/* 0 is subnormal, m * 2^-9; the pattern with all exponent and mantissa     */
/* bits set is NaN, there is no inf).                                       */
/* ------------------------------------------------------------------------ */
static inline double e4m3_value(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return (c & 0x80) ? -v : v;
}

/* IEEE binary16: sign, 5 exponent bits with bias 15, 10 mantissa bits;     */
/* exponent 0 holds the subnormals m * 2^-24; exponent 31 is inf / NaN.     */
static inline double f16_value(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -24);
  else v = ldexp(1.0 + m / 1024.0, e - 15);
  return (h & 0x8000) ? -v : v;
}

static inline double ref_elem(const void* X, int dtype, int64_t row, int32_t d, int32_t t) {
  if (dtype == 0) return (double)((const float*)X)[row * (int64_t)d + t];
  if (dtype == 2) return (double)((const int8_t*)X)[row * (int64_t)d + t];  /* int8 codes */
  if (dtype == 3) return e4m3_value(((const uint8_t*)X)[row * (int64_t)d + t]);
  if (dtype == 4) return f16_value(((const uint16_t*)X)[row * (int64_t)d + t]);
  if (dtype == 5) return (double)((const uint8_t*)X)[row * (int64_t)d + t];     /* uint8 */
  uint32_t bits = (uint32_t)((const uint16_t*)X)[row * (int64_t)d + t] << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* Nearest centroid by brute force: for each selected row, the squared       */
/* distance to every centroid, written out as the sum over coordinates; ties */
/* go to the lowest index. Also returns the runner-up distance (used by the  */
/* tests to tell decided labels from near-ties).                             */
void ref_assign(const void* X, int dtype, int64_t nrows, const int64_t* rows, int32_t d,
                const float* C, int32_t k, int32_t* labels, double* d1, double* d2,
                int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
    for (int64_t i = 0; i < nrows; ++i) {
      int64_t row = rows ? rows[i] : i;
      for (int32_t t = 0; t < d; ++t) x[t] = ref_elem(X, dtype, row, d, t);
      double best = INFINITY, second = INFINITY;
      int32_t arg = -1;
      int32_t j = 0;
      /* four centroids at a time, each distance summed over t in order as in
         the single-centroid loop below (identical results, more ILP) */
      for (; j + 4 <= k; j += 4) {
        const float* c0 = C + (int64_t)j * d;
        const float* c1 = c0 + d;
        const float* c2 = c1 + d;
        const float* c3 = c2 + d;
        double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
        for (int32_t t = 0; t < d; ++t) {
          const double a0 = x[t] - (double)c0[t], a1 = x[t] - (double)c1[t];
          const double a2 = x[t] - (double)c2[t], a3 = x[t] - (double)c3[t];
          s0 += a0 * a0;
          s1 += a1 * a1;
          s2 += a2 * a2;
          s3 += a3 * a3;
        }
        const double sv[4] = {s0, s1, s2, s3};
        for (int q = 0; q < 4; ++q) {
          if (sv[q] < best) {
            second = best;
            best = sv[q];
            arg = j + q;
          } else if (sv[q] < second) {
            second = sv[q];
          }
        }
      }
      for (; j < k; ++j) {
        const float* c = C + (int64_t)j * d;
        double s = 0.0;
        for (int32_t t = 0; t < d; ++t) {
          double diff = x[t] - (double)c[t];
          s += diff * diff;
        }
        if (s < best) {
          second = best;
          best = s;
          arg = j;
        } else if (s < second) {
          second = s;
        }
      }
      labels[i] = arg;
      d1[i] = best;
      if (d2) d2[i] = second;
    }
    free(x);
  }
}

/* Squared distance of each selected row to one given centroid each.        */
void ref_dist_to(const void* X, int dtype, int64_t nrows, const int64_t* rows, int32_t d,
                 const float* C, const int32_t* labels, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t row = rows ? rows[i] : i;
    const float* c = C + (int64_t)labels[i] * d;
    double s = 0.0;
    for (int32_t t = 0; t < d; ++t) {
      double diff = ref_elem(X, dtype, row, d, t) - (double)c[t];
      s += diff * diff;
    }
    out[i] = s;
  }
}

/* Spherical e-means (README "Spherical e-means"): each row goes to the      */
/* centroid of largest dot product, the lowest index on ties. Returns       */
/* the label, the best and the runner-up dot product (fp64, summed over t in */
/* order).                                                                    */
void ref_assign_ip(const void* X, int dtype, int64_t nrows, const int64_t* rows, int32_t d,
                   const float* C, int32_t k, int32_t* labels, double* s1, double* s2,
                   int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
    for (int64_t i = 0; i < nrows; ++i) {
      int64_t row = rows ? rows[i] : i;
      for (int32_t t = 0; t < d; ++t) x[t] = ref_elem(X, dtype, row, d, t);
      double best = -INFINITY, second = -INFINITY;
      int32_t arg = -1;
      for (int32_t j = 0; j < k; ++j) {
        const float* c = C + (int64_t)j * d;
        double s = 0.0;
        for (int32_t t = 0; t < d; ++t) s += x[t] * (double)c[t];
        if (s > best) {
          second = best;
          best = s;
          arg = j;
        } else if (s > second) {
          second = s;
        }
      }
      labels[i] = arg;
      s1[i] = best;
      s2[i] = second;
    }
    free(x);
  }
}

/* Dot product of each selected row with the centroid of the given label.     */
void ref_dot_to(const void* X, int dtype, int64_t nrows, const int64_t* rows, int32_t d,
                const float* C, const int32_t* labels, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t row = rows ? rows[i] : i;
    const float* c = C + (int64_t)labels[i] * d;
    double s = 0.0;
    for (int32_t t = 0; t < d; ++t) s += ref_elem(X, dtype, row, d, t) * (double)c[t];
    out[i] = s;
  }
}

/* Per-cluster count and sum of the selected rows, in fp64. Each cluster's  */
/* sum is taken in row order (the order of a sequential loop over the rows);  */
/* rows are bucketed by label first only so clusters can run in parallel.     */
void ref_group(const void* X, int dtype, int64_t nrows, const int64_t* rows,
               const int32_t* labels, int32_t d, int32_t k, double* sums, int64_t* counts) {
  memset(counts, 0, sizeof(int64_t) * (size_t)k);
  for (int64_t i = 0; i < nrows; ++i) counts[labels[i]] += 1;
  int64_t* start = (int64_t*)malloc(sizeof(int64_t) * ((size_t)k + 1));
  int64_t* cursor = (int64_t*)malloc(sizeof(int64_t) * (size_t)k);
  int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrows > 0 ? nrows : 1));
  start[0] = 0;
  for (int32_t j = 0; j < k; ++j) start[j + 1] = start[j] + counts[j];
  for (int32_t j = 0; j < k; ++j) cursor[j] = start[j];
  for (int64_t i = 0; i < nrows; ++i) order[cursor[labels[i]]++] = i;
#pragma omp parallel for schedule(dynamic, 16)
  for (int32_t j = 0; j < k; ++j) {
    double* s = sums + (int64_t)j * d;
    for (int32_t t = 0; t < d; ++t) s[t] = 0.0;
    for (int64_t p = start[j]; p < start[j + 1]; ++p) {
      int64_t row = rows ? rows[order[p]] : order[p];
      for (int32_t t = 0; t < d; ++t) s[t] += ref_elem(X, dtype, row, d, t);
    }
  }
  free(order);
  free(cursor);
  free(start);
}

/* ======================================================================== */
/* Host-pointer mirrors of the library's boundary: emeans_ref_recipe,       */
/* emeans_ref_assign and emeans_ref_train. They take the same steps as the  */
/* Python oracle (oracle/__init__.py: recipe, assign, train with default    */
/* options) for fp32 data, in the same arithmetic:                          */
/*   recipe  - scaling laws (faiss e_means README, "Scaling laws"): batch   */
/*             size c * k^0.134749 * n^0.876473 * T^0.813344 rounded to the */
/*             nearest power of two and capped at the largest power of two  */
/*             <= n / 2; alpha0 = 0.8244 k^-0.4617 B^0.9003 n^-0.4498       */
/*             T^-0.1057 clamped to [1e-4, 1]; floor(T) full passes plus    */
/*             floor(frac(T) n) rows; revival threshold 0.1 (0 for d <= 2); */
/*   assign  - the nearest centroid in fp64, ties to the lowest index;      */
/*   train   - the batch loop of the README's "Data too big for memory"     */
/*             rules: a fresh keyed order every pass, N <- fl(fl(b N) +      */
/*             fl(a n)) in fp32 with b = fl(1 - a), S <- (b S + a s) in     */
/*             fp64 stored fp32, c = S / N where N > 0, revival after every */
/*             fifth step (blog, third change), and the closing exact mean  */
/*             of the last pass (README "How the centroid updates work").   */
/* Return 0, or -1 for arguments outside the library's own bounds (the      */
/* outputs are then untouched).                                             */
/* ======================================================================== */
enum { REF_LAW_THROUGHPUT = 1, REF_LAW_QUALITY = 2 };

int emeans_ref_recipe(int64_t n, int32_t d, int32_t k, double T, int64_t* batch_size,
                      double* alpha0, int32_t* passes, int64_t* total_steps, double* threshold) {
  if (n < 1 || d < 1 || k < 1 || k > n || !(T > 0.0)) return -1;
  const int law = d <= 16 ? REF_LAW_QUALITY : REF_LAW_THROUGHPUT;
  const double c = law == REF_LAW_QUALITY ? 0.00439175 : 0.035134;
  const double braw = c * pow((double)k, 0.134749) * pow((double)n, 0.876473) * pow(T, 0.813344);
  int64_t B = (int64_t)ldexp(1.0, (int)floor(log2(braw) + 0.5));
  const int64_t cap = n >= 2 ? (int64_t)ldexp(1.0, (int)floor(log2((double)n / 2.0))) : 1;
  if (B > cap) B = cap;
  if (B < 1) B = 1;
  double a0 = 0.8244 * pow((double)k, -0.4617) * pow((double)B, 0.9003) *
              pow((double)n, -0.4498) * pow(T, -0.1057);
  if (a0 < 1e-4) a0 = 1e-4;
  if (a0 > 1.0) a0 = 1.0;
  const int full = (int)floor(T);
  const int64_t frac_rows = (int64_t)floor((T - full) * (double)n);
  int np_ = full + (frac_rows > 0 ? 1 : 0);
  int64_t steps = (int64_t)full * ((n + B - 1) / B) + (frac_rows > 0 ? (frac_rows + B - 1) / B : 0);
  if (batch_size) *batch_size = B;
  if (alpha0) *alpha0 = a0;
  if (passes) *passes = np_;
  if (total_steps) *total_steps = steps;
  if (threshold) *threshold = d <= 2 ? 0.0 : 0.1;
  return 0;
}

int emeans_ref_assign(const float* X, int64_t n, int32_t d, const float* C, int32_t k,
                      int32_t* labels, float* dists) {
  if (n < 0 || d < 1 || k < 1 || !X || !C || !labels) return -1;
  double* d1 = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  ref_assign(X, 0, n, NULL, d, C, k, labels, d1, NULL, 0);
  if (dists)
    for (int64_t i = 0; i < n; ++i) dists[i] = (float)d1[i];
  free(d1);
  return 0;
}

/* Revival after step t (the Python oracle's _revive, euclidean mode). */
static int64_t ref_revive(int64_t t, uint64_t seed, double thr, int32_t k, int32_t d, float* N,
                          float* S, float* C) {
  double total = 0.0;
  for (int32_t j = 0; j < k; ++j) total += (double)N[j];
  const double th = thr * (total / (double)k);
  unsigned char* live = (unsigned char*)malloc((size_t)k);
  double* cum = (double*)malloc(sizeof(double) * (size_t)k);
  int32_t last_live = -1;
  for (int32_t j = 0; j < k; ++j) {
    live[j] = !((double)N[j] < th);
    if (live[j]) last_live = j;
  }
  int64_t splits = 0;
  const float eps = (float)ldexp(1.0, -10);
  for (int32_t j = 0; j < k; ++j) {
    if (live[j]) continue;
    /* u from Philox stream 3: 53 random bits in [0, 1) */
    const uint64_t ctr[4] = {(uint64_t)j, (uint64_t)t, 0, 3}, key[2] = {seed, 0};
    uint64_t w[4];
    ref_philox4x64(ctr, key, w);
    const double u = (double)(w[0] >> 11) * ldexp(1.0, -53);
    double run = 0.0;
    for (int32_t q = 0; q < k; ++q) {
      run += live[q] ? (double)N[q] : 0.0;
      cum[q] = run;
    }
    const double target = u * cum[k - 1];
    int32_t i = k;
    for (int32_t q = 0; q < k; ++q)
      if (cum[q] > target) {
        i = q;
        break;
      }
    if (i >= k || !live[i]) i = last_live;
    const float* si = S + (int64_t)i * d;
    float* sj = S + (int64_t)j * d;
    float* sim = S + (int64_t)i * d;
    N[i] = N[i] * 0.5f;
    N[j] = N[i];
    for (int32_t e = 0; e < d; ++e) {
      /* sign of coordinate e: bit e % 64 of word (e / 64) % 4 of the Philox
         stream-4 block with counter word 2 = e / 256; a set bit means -1 */
      const uint64_t c4[4] = {(uint64_t)j, (uint64_t)t, (uint64_t)(e / 256), 4};
      uint64_t sw[4];
      ref_philox4x64(c4, key, sw);
      const float sg = ((sw[(e / 64) % 4] >> (e % 64)) & 1ULL) ? -1.0f : 1.0f;
      const float half = si[e] * 0.5f;
      const float pe = eps * sg;
      sj[e] = half * (1.0f + pe);
      sim[e] = half * (1.0f - pe);
    }
    for (int32_t e = 0; e < d; ++e) {
      C[(int64_t)i * d + e] = (float)((double)S[(int64_t)i * d + e] / (double)N[i]);
      C[(int64_t)j * d + e] = (float)((double)S[(int64_t)j * d + e] / (double)N[j]);
    }
    ++splits;
  }
  free(cum);
  free(live);
  return splits;
}

int emeans_ref_train(const float* X, int64_t n, int32_t d, int32_t k, double T, uint64_t seed,
                     float* centroids, int32_t* labels, int64_t* n_splits) {
  int64_t B, S_tot;
  double a0, thr;
  int32_t npass;
  if (!X || !centroids || emeans_ref_recipe(n, d, k, T, &B, &a0, &npass, &S_tot, &thr)) return -1;
  const size_t kd = (size_t)k * (size_t)d;
  float* C = centroids;
  float* N = (float*)calloc((size_t)k, sizeof(float));
  float* S = (float*)calloc(kd, sizeof(float));
  int64_t* LN = (int64_t*)calloc((size_t)k, sizeof(int64_t));
  double* LS = (double*)calloc(kd, sizeof(double));
  int64_t* counts = (int64_t*)malloc(sizeof(int64_t) * (size_t)k);
  double* sums = (double*)malloc(sizeof(double) * kd);
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)B);
  int32_t* lab = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  double* d1 = (double*)malloc(sizeof(double) * (size_t)B);
  /* starting centroids: the first k entries of the init order (stream 1) */
  int64_t* init = (int64_t*)malloc(sizeof(int64_t) * (size_t)k);
  ref_perm_range((uint64_t)n, seed, 1, 0, 0, (uint64_t)k, init);
  for (int32_t j = 0; j < k; ++j) memcpy(C + (size_t)j * d, X + (size_t)init[j] * d, sizeof(float) * d);
  free(init);
  if (labels)
    for (int64_t r = 0; r < n; ++r) labels[r] = -1;
  const int full = (int)floor(T);
  int64_t t = 0, splits = 0;
  for (int32_t e = 0; e < npass; ++e) {
    const int64_t rows_e = e < full ? n : (int64_t)floor((T - full) * (double)n);
    const int last = e == npass - 1;
    for (int64_t s0 = 0; s0 < rows_e; s0 += B) {
      const int64_t Bt = rows_e - s0 < B ? rows_e - s0 : B;
      ref_perm_range((uint64_t)n, seed, 2, (uint64_t)e, (uint64_t)s0, (uint64_t)Bt, rows);
      ref_assign(X, 0, Bt, rows, d, C, k, lab, d1, NULL, 0);
      ref_group(X, 0, Bt, rows, lab, d, k, sums, counts);
      /* cosine step: alpha0 (0.1 + 0.45 (1 + cos(pi t / (S - 1)))), in fp32 */
      const float a = S_tot == 1 ? (float)a0
                                 : (float)(a0 * (0.1 + 0.45 * (1.0 + cos(M_PI * (double)t /
                                                                          (double)(S_tot - 1)))));
      const float b = 1.0f - a;
      for (int32_t j = 0; j < k; ++j) {
        N[j] = (b * N[j]) + (a * (float)counts[j]);
        for (int32_t q = 0; q < d; ++q) {
          const size_t ix = (size_t)j * d + q;
          S[ix] = (float)((double)b * (double)S[ix] + (double)a * sums[ix]);
        }
        if (N[j] > 0.0f)
          for (int32_t q = 0; q < d; ++q) {
            const size_t ix = (size_t)j * d + q;
            C[ix] = (float)((double)S[ix] / (double)N[j]);
          }
      }
      if (last) {
        for (int32_t j = 0; j < k; ++j) LN[j] += counts[j];
        for (size_t ix = 0; ix < kd; ++ix) LS[ix] += sums[ix];
        if (labels)
          for (int64_t r = 0; r < Bt; ++r) labels[rows[r]] = lab[r];
      }
      if (thr > 0.0 && (t + 1) % 5 == 0) splits += ref_revive(t, seed, thr, k, d, N, S, C);
      ++t;
    }
  }
  /* closing step: the exact mean of each cluster's rows in the last pass */
  for (int32_t j = 0; j < k; ++j)
    if (LN[j] > 0)
      for (int32_t q = 0; q < d; ++q) {
        const size_t ix = (size_t)j * d + q;
        C[ix] = (float)(LS[ix] / (double)LN[j]);
      }
  if (n_splits) *n_splits = splits;
  free(d1);
  free(lab);
  free(rows);
  free(sums);
  free(counts);
  free(LS);
  free(LN);
  free(S);
  free(N);
  return 0;
}
