// C ABI of libemeans.so: argument checks, the scaling-law recipe, workspace
// and the stream-ordered step loop of e-means training.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <chrono>
#include <string>
#include <vector>

#include "emeans.h"
#include "kernels.hpp"

using namespace emk;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess) {                                                               \
      rc = fail(e_ == hipErrorOutOfMemory ? EMEANS_ENOMEM : EMEANS_EHIP, "%s: %s (%s:%d)", \
                #expr, hipGetErrorString(e_), __FILE__, __LINE__);                        \
      goto done;                                                                          \
    }                                                                                     \
  } while (0)

constexpr int kGroupRows = 64;   // rows per grouping work item
constexpr int kReviveEvery = 5;  // blog: dead clusters are checked every five batches

struct Recipe {
  int law = 0;
  int64_t B = 0;
  double alpha0 = 0;
  double thr = 0;
  int npass = 0;
  int64_t rows[EMEANS_MAX_PASSES] = {};
  int64_t steps[EMEANS_MAX_PASSES] = {};
  int64_t S = 0;
};

// README "Scaling laws" (1)-(3) with their constraints; "Parameters" note on
// low dimension; "Manual overrides"; "Settings" (unused_threshold).
int make_recipe(int64_t n, int32_t d, int32_t k, double T, const emeans_opts* o, Recipe& r) {
  if (n < 1) return fail(EMEANS_EINVAL, "n must be >= 1 (got %lld)", (long long)n);
  if (d < 1) return fail(EMEANS_EINVAL, "d must be >= 1 (got %d)", d);
  if (k < 1) return fail(EMEANS_EINVAL, "k must be >= 1 (got %d)", k);
  if ((int64_t)k > n) return fail(EMEANS_EINVAL, "k (%d) must not exceed n (%lld)", k, (long long)n);
  if (!(T > 0.0) || !isfinite(T)) return fail(EMEANS_EINVAL, "T must be > 0 (got %g)", T);
  const int32_t law_opt = o ? o->batch_law : 0;
  if (law_opt < 0 || law_opt > 2) return fail(EMEANS_EINVAL, "batch_law must be 0, 1 or 2");
  r.law = law_opt ? law_opt : (d <= 16 ? EMEANS_LAW_QUALITY : EMEANS_LAW_THROUGHPUT);
  const int64_t bs = o ? o->batch_size : 0;
  if (bs < 0) return fail(EMEANS_EINVAL, "batch_size must be >= 0");
  if (bs > 0) {
    r.B = bs < n ? bs : n;
  } else {
    const double c = r.law == EMEANS_LAW_QUALITY ? 0.00439175 : 0.035134;
    const double braw = c * pow((double)k, 0.134749) * pow((double)n, 0.876473) * pow(T, 0.813344);
    const int e = (int)floor(log2(braw) + 0.5);
    int64_t B = e <= 0 ? 1 : (e >= 62 ? ((int64_t)1 << 62) : ((int64_t)1 << e));
    int64_t cap = 1;
    if (n >= 2) {
      const int ce = (int)floor(log2((double)n / 2.0));
      cap = ce <= 0 ? 1 : ((int64_t)1 << ce);
    }
    if (B > cap) B = cap;
    if (B < 1) B = 1;
    r.B = B;
  }
  const double a0 = o ? o->alpha0 : 0.0;
  if (a0 < 0 || !isfinite(a0)) return fail(EMEANS_EINVAL, "alpha0 must be >= 0");
  if (a0 > 0) {
    r.alpha0 = a0;
  } else {
    double a = 0.8244 * pow((double)k, -0.4617) * pow((double)r.B, 0.9003) *
               pow((double)n, -0.4498) * pow(T, -0.1057);
    r.alpha0 = a < 1e-4 ? 1e-4 : (a > 1.0 ? 1.0 : a);
  }
  const double ut = o ? o->unused_threshold : 0.0;
  if (!isfinite(ut)) return fail(EMEANS_EINVAL, "unused_threshold must be finite");
  r.thr = ut == 0.0 ? (d <= 2 ? 0.0 : 0.1) : (ut < 0.0 ? 0.0 : ut);
  if (r.thr >= 1.0) return fail(EMEANS_EINVAL, "unused_threshold must be < 1");
  const int64_t full = (int64_t)floor(T);
  const int64_t frac_rows = (int64_t)floor((T - (double)full) * (double)n);
  const int64_t np = full + (frac_rows > 0 ? 1 : 0);
  if (np > EMEANS_MAX_PASSES || np < 1)
    return fail(EMEANS_EINVAL, "T gives %lld passes (1..%d supported)", (long long)np,
                EMEANS_MAX_PASSES);
  r.npass = (int)np;
  r.S = 0;
  for (int e = 0; e < r.npass; ++e) {
    r.rows[e] = e < full ? n : frac_rows;
    r.steps[e] = (r.rows[e] + r.B - 1) / r.B;
    r.S += r.steps[e];
  }
  return EMEANS_OK;
}

void fill_stats(const Recipe& r, emeans_stats* s) {
  memset(s, 0, sizeof *s);
  s->batch_size = r.B;
  s->total_steps = r.S;
  s->alpha0 = r.alpha0;
  s->unused_threshold = r.thr;
  s->law = r.law;
  s->n_passes = r.npass;
  for (int e = 0; e < r.npass; ++e) {
    s->rows_per_pass[e] = r.rows[e];
    s->steps_per_pass[e] = r.steps[e];
  }
}

// Cosine decay from alpha0 at the first update step to alpha0/10 at the last
// (blog, second change; README "How the centroid updates work").
float alpha_at(double alpha0, int64_t t, int64_t S) {
  if (S <= 1) return (float)alpha0;
  const double a = alpha0 * (0.1 + 0.45 * (1.0 + cos(M_PI * (double)t / (double)(S - 1))));
  return (float)a;
}

int check_device(const void* p, const char* name) {
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof attr);
  const hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(EMEANS_ENOTDEVICE, "%s is not a device pointer (%s)", name, hipGetErrorString(e));
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(EMEANS_ENOTDEVICE, "%s is not device memory", name);
  return EMEANS_OK;
}

// Bump allocator over one stream-ordered allocation.
struct Arena {
  size_t used = 0;
  std::vector<std::pair<void**, size_t>> wants;
  template <typename T>
  void want(T** p, size_t count) {
    wants.push_back({reinterpret_cast<void**>(p), count * sizeof(T)});
  }
  hipError_t alloc(void** base, hipStream_t st) {
    size_t total = 0;
    for (auto& w : wants) total += (w.second + 255) & ~(size_t)255;
    if (total == 0) total = 256;
    hipError_t e = hipMallocAsync(base, total, st);
    if (e != hipSuccess) return e;
    size_t off = 0;
    for (auto& w : wants) {
      *w.first = static_cast<char*>(*base) + off;
      off += (w.second + 255) & ~(size_t)255;
    }
    used = total;
    return hipSuccess;
  }
};

}  // namespace

extern "C" {

const char* emeans_last_error(void) { return g_err.c_str(); }

int emeans_version(void) { return 100; }

int emeans_recipe(int64_t n, int32_t d, int32_t k, double T, const emeans_opts* opts,
                  emeans_stats* out) {
  g_err.clear();
  if (!out) return fail(EMEANS_EINVAL, "out is NULL");
  Recipe r;
  const int rc = make_recipe(n, d, k, T, opts, r);
  if (rc) return rc;
  fill_stats(r, out);
  return EMEANS_OK;
}

int emeans_batch_rows(int64_t n, uint64_t seed, int32_t pass, int64_t start, int64_t count,
                      int32_t* rows_out, void* stream) {
  g_err.clear();
  if (n < 1 || n >= ((int64_t)1 << 31)) return fail(EMEANS_EINVAL, "n out of range");
  if (pass < 0 || start < 0 || count < 0 || start + count > n)
    return fail(EMEANS_EINVAL, "slot range [%lld, %lld) outside [0, %lld)", (long long)start,
                (long long)(start + count), (long long)n);
  if (!rows_out) return fail(EMEANS_EINVAL, "rows_out is NULL");
  int rc = check_device(rows_out, "rows_out");
  if (rc) return rc;
  const PermKey pk = make_perm_key((uint64_t)n, seed, kStreamPerm, (uint64_t)pass);
  const hipError_t e = launch_sample_rows_i32(pk, (uint64_t)start, (int)count, rows_out,
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EMEANS_EHIP, "sampler launch: %s", hipGetErrorString(e));
  return EMEANS_OK;
}

int emeans_assign(const void* X, int64_t n, int32_t d, const float* C, int32_t k,
                  int32_t* labels, float* dists, const emeans_opts* opts) {
  g_err.clear();
  const int32_t dtype = opts ? opts->dtype : EMEANS_F32;
  if (dtype != EMEANS_F32 && dtype != EMEANS_BF16)
    return fail(EMEANS_EDTYPE, "dtype %d not supported (fp32 = 0, bf16 = 1)", dtype);
  if (n < 0 || n >= ((int64_t)1 << 31)) return fail(EMEANS_EINVAL, "n out of range (%lld)", (long long)n);
  if (d < 1) return fail(EMEANS_EINVAL, "d must be >= 1");
  if (k < 1) return fail(EMEANS_EINVAL, "k must be >= 1");
  if (!X || !C || !labels) return fail(EMEANS_EINVAL, "X, C and labels must not be NULL");
  if (n == 0) return EMEANS_OK;
  int rc;
  if ((rc = check_device(X, "X")) || (rc = check_device(C, "C")) ||
      (rc = check_device(labels, "labels")) || (dists && (rc = check_device(dists, "dists"))))
    return rc;
  hipStream_t st = static_cast<hipStream_t>(opts ? opts->stream : nullptr);
  const bool bf16 = dtype == EMEANS_BF16;
  const bool bsearch = !bf16 && opts && opts->bf16_search;  // fp32 rows searched in bf16
  const bool sph = opts && opts->spherical;  // highest dot product, similarity out
  void* base = nullptr;
  float* bias = nullptr;
  uint16_t* chat = nullptr;
  uint16_t* xb = nullptr;
  Arena ar;
  ar.want(&bias, (size_t)k);
  if (bf16 || bsearch) ar.want(&chat, (size_t)k * d);
  if (bsearch) ar.want(&xb, (size_t)n * d);
  rc = EMEANS_OK;
  HIP_TRY(ar.alloc(&base, st));
  HIP_TRY(launch_prep(C, k, d, bias, chat, sph, st));
  if (bsearch) HIP_TRY(launch_cast_rows(static_cast<const float*>(X), d, nullptr, (int)n, xb, st));
  HIP_TRY(launch_assign(bf16 || bsearch, bsearch ? (const void*)xb : X, d, nullptr, (int)n,
                        (bf16 || bsearch) ? (const void*)chat : (const void*)C, bias, k, labels,
                        dists, nullptr, nullptr, sph, st));
done:
  if (base) {
    const hipError_t e = hipFreeAsync(base, st);
    if (e != hipSuccess && rc == EMEANS_OK)
      rc = fail(EMEANS_EHIP, "hipFreeAsync: %s", hipGetErrorString(e));
  }
  return rc;
}

int emeans_train(const void* X, int64_t n, int32_t d, int32_t k, double T, uint64_t seed,
                 float* centroids, int32_t* labels, const emeans_opts* opts,
                 emeans_stats* stats) {
  g_err.clear();
  const auto t_start = std::chrono::steady_clock::now();
  const int32_t dtype = opts ? opts->dtype : EMEANS_F32;
  if (dtype != EMEANS_F32 && dtype != EMEANS_BF16)
    return fail(EMEANS_EDTYPE, "dtype %d not supported (fp32 = 0, bf16 = 1)", dtype);
  Recipe r;
  int rc = make_recipe(n, d, k, T, opts, r);
  if (rc) return rc;
  if (n >= ((int64_t)1 << 31)) return fail(EMEANS_EINVAL, "n must be < 2^31");
  if (r.B >= ((int64_t)1 << 24))
    return fail(EMEANS_EINVAL, "batch size must be < 2^24 (counts are exact in fp32)");
  if (!X || !centroids) return fail(EMEANS_EINVAL, "X and centroids must not be NULL");
  if ((rc = check_device(X, "X")) || (rc = check_device(centroids, "centroids")) ||
      (labels && (rc = check_device(labels, "labels"))))
    return rc;
  if (opts && opts->trace_labels && (rc = check_device(opts->trace_labels, "trace_labels")))
    return rc;
  if (opts && opts->out_counts && (rc = check_device(opts->out_counts, "out_counts"))) return rc;
  if (opts && opts->split_log && opts->split_log_cap < 0)
    return fail(EMEANS_EINVAL, "split_log_cap must be >= 0");

  hipStream_t st = static_cast<hipStream_t>(opts ? opts->stream : nullptr);
  const bool bf16 = dtype == EMEANS_BF16;
  // fp32 rows searched in bf16: each batch is gathered and rounded into xb
  const bool bsearch = !bf16 && opts && opts->bf16_search;
  const bool sbf = bf16 || bsearch;  // the search runs in bf16 against chat
  const bool sph = opts && opts->spherical;  // spherical e-means
  const bool profile = opts && opts->profile;
  const size_t kd = (size_t)k * d;
  const int64_t B = r.B;
  const int64_t log_cap = (opts && opts->split_log) ? opts->split_log_cap : 0;

  void* base = nullptr;
  uint32_t *rows = nullptr, *order = nullptr;
  int32_t *blab = nullptr, *counts = nullptr, *cursor = nullptr, *off = nullptr,
          *ovf_n = nullptr, *pass_counts = nullptr, *flags = nullptr, *dead = nullptr,
          *dlog = nullptr, *pair_i = nullptr, *rv_pos = nullptr, *rv_head = nullptr,
          *rv_cbase = nullptr, *rv_clen = nullptr, *rv_heads = nullptr, *rv_list = nullptr,
          *rv_nheads = nullptr;
  double* rv_u = nullptr;
  int2* ovf = nullptr;
  float *bdist = nullptr, *s_acc = nullptr, *S = nullptr, *N = nullptr, *LS = nullptr,
        *bias = nullptr, *n0 = nullptr, *pair_n = nullptr;
  uint16_t *chat = nullptr, *xb = nullptr;
  // per pass: [0, P) sum of distances, [P, 3P) sum n^2 and sum n, [3P, 4P) splits (int64)
  double* dstat = nullptr;
  int64_t* counters = nullptr;
  struct Span {
    int cls;
    hipEvent_t a, b;
  };
  std::vector<Span> spans;
  double host_stat[4 * EMEANS_MAX_PASSES];
  int64_t host_counters[4] = {0, 0, 0, 0};
  int64_t trace_off = 0;
  int64_t t = 0;

  Arena ar;
  ar.want(&rows, (size_t)B);
  ar.want(&order, (size_t)B);
  ar.want(&blab, (size_t)B);
  ar.want(&bdist, (size_t)B);
  ar.want(&counts, (size_t)k);
  ar.want(&cursor, (size_t)k);
  ar.want(&off, (size_t)k + 1);
  ar.want(&ovf, (size_t)(B / kGroupRows) + 1);
  ar.want(&ovf_n, 1);
  ar.want(&pass_counts, (size_t)k);
  ar.want(&flags, (size_t)k);
  ar.want(&dead, (size_t)k);
  ar.want(&n0, (size_t)k);
  ar.want(&pair_i, (size_t)k);
  ar.want(&pair_n, (size_t)k);
  ar.want(&rv_u, (size_t)k);
  ar.want(&rv_pos, (size_t)k);
  ar.want(&rv_head, (size_t)k);
  ar.want(&rv_cbase, (size_t)k);
  ar.want(&rv_clen, (size_t)k);
  ar.want(&rv_heads, (size_t)k);
  ar.want(&rv_list, (size_t)k);
  ar.want(&rv_nheads, 1);
  ar.want(&s_acc, kd);
  ar.want(&S, kd);
  ar.want(&N, (size_t)k);
  ar.want(&LS, kd);
  ar.want(&bias, (size_t)k);
  if (sbf) ar.want(&chat, kd);
  if (bsearch) ar.want(&xb, (size_t)B * d);
  ar.want(&dstat, (size_t)4 * EMEANS_MAX_PASSES);
  ar.want(&counters, 4);
  if (log_cap > 0) ar.want(&dlog, (size_t)3 * log_cap);

  // Device time of a kernel class: events recorded on the launch stream around it.
  enum { kAssign = 0, kBucket, kGroup, kUpdate, kRevive, kSample, kClasses };
  auto timed = [&](int cls, auto&& launch) -> hipError_t {
    if (!profile) return launch();
    Span sp{cls, nullptr, nullptr};
    hipError_t er = hipEventCreate(&sp.a);
    if (er == hipSuccess) er = hipEventCreate(&sp.b);
    if (er != hipSuccess) return er;
    spans.push_back(sp);
    if ((er = hipEventRecord(sp.a, st)) != hipSuccess) return er;
    if ((er = launch()) != hipSuccess) return er;
    return hipEventRecord(sp.b, st);
  };
  const int64_t max_steps = opts ? opts->max_steps : 0;
  if (max_steps < 0) return fail(EMEANS_EINVAL, "max_steps must be >= 0");
  const int64_t run_steps = (max_steps > 0 && max_steps < r.S) ? max_steps : r.S;
  bool last_pass_begun = false;

  HIP_TRY(ar.alloc(&base, st));
  // zero the statistics and every accumulator the step loop expects at zero
  HIP_TRY(hipMemsetAsync(counts, 0, sizeof(int32_t) * k, st));
  HIP_TRY(hipMemsetAsync(pass_counts, 0, sizeof(int32_t) * k, st));
  HIP_TRY(hipMemsetAsync(s_acc, 0, sizeof(float) * kd, st));
  HIP_TRY(hipMemsetAsync(S, 0, sizeof(float) * kd, st));
  HIP_TRY(hipMemsetAsync(N, 0, sizeof(float) * k, st));
  HIP_TRY(hipMemsetAsync(LS, 0, sizeof(float) * kd, st));
  HIP_TRY(hipMemsetAsync(dstat, 0, sizeof(double) * 4 * EMEANS_MAX_PASSES, st));
  HIP_TRY(hipMemsetAsync(counters, 0, sizeof(int64_t) * 4, st));
  if (labels) HIP_TRY(hipMemsetAsync(labels, 0xFF, sizeof(int32_t) * (size_t)n, st));

  // starting centroids: k distinct rows (first k entries of the init permutation)
  HIP_TRY(launch_init_centroids(bf16, X, d, make_perm_key((uint64_t)n, seed, kStreamInit, 0), k,
                                centroids, sph, st));
  HIP_TRY(launch_prep(centroids, k, d, bias, chat, sph, st));

  for (int e = 0; e < r.npass && t < run_steps; ++e) {
    const bool last = e == r.npass - 1;
    last_pass_begun = last;
    const PermKey pk = make_perm_key((uint64_t)n, seed, kStreamPerm, (uint64_t)e);
    for (int64_t s = 0; s < r.steps[e] && t < run_steps; ++s, ++t) {
      const int64_t rem = r.rows[e] - s * B;
      const int nb = (int)(rem < B ? rem : B);
      const float a = alpha_at(r.alpha0, t, r.S);
      const float b = 1.0f - a;
      HIP_TRY(timed(kSample, [&] {
        hipError_t er = launch_sample_rows(pk, (uint64_t)(s * B), nb, rows, st);
        if (er != hipSuccess || !bsearch) return er;
        return launch_cast_rows(static_cast<const float*>(X), d, rows, nb, xb, st);
      }));
      HIP_TRY(timed(kAssign, [&] {
        if (bsearch)
          return launch_assign(true, xb, d, nullptr, nb, chat, bias, k, blab, bdist, counts,
                               dstat + e, sph, st);
        return launch_assign(bf16, X, d, rows, nb, bf16 ? (const void*)chat : (const void*)centroids,
                             bias, k, blab, bdist, counts, dstat + e, sph, st);
      }));
      if (opts && opts->trace_labels) {
        HIP_TRY(hipMemcpyAsync(opts->trace_labels + trace_off, blab, sizeof(int32_t) * nb,
                               hipMemcpyDeviceToDevice, st));
        trace_off += nb;
      }
      HIP_TRY(timed(kBucket, [&] {
        hipError_t er = launch_scan(counts, k, kGroupRows, off, cursor, ovf, ovf_n, st);
        if (er != hipSuccess) return er;
        return launch_scatter(blab, rows, nb, cursor, order, (last && labels) ? labels : nullptr, st);
      }));
      HIP_TRY(timed(kGroup, [&] {
        return launch_group(bf16, X, d, order, off, ovf, ovf_n, k, kGroupRows, nb, s_acc, st);
      }));
      HIP_TRY(timed(kUpdate, [&] {
        return launch_ema(k, d, a, b, counts, s_acc, N, S, centroids, bias, chat, pass_counts,
                          last ? LS : nullptr, sph, st);
      }));
      if (r.thr > 0.0 && (t + 1) % kReviveEvery == 0) {
        ReviveArgs ra{k, d, N, S, centroids, bias, chat, r.thr, seed, (uint64_t)t, flags, dead,
                      n0, rv_u, pair_i, pair_n, rv_pos, rv_head, rv_cbase, rv_clen, rv_heads,
                      rv_list, rv_nheads, counters, dlog, log_cap, 0, sph ? 1 : 0};
        HIP_TRY(timed(kRevive, [&] { return launch_revive(ra, st); }));
      }
    }
    HIP_TRY(launch_pass_stats(pass_counts, k, dstat + EMEANS_MAX_PASSES + 2 * e, last ? 0 : 1, st));
    // per-pass split count: snapshot counters[3] then reset it
    HIP_TRY(hipMemcpyAsync(dstat + 3 * EMEANS_MAX_PASSES + e, counters + 3, sizeof(int64_t),
                           hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemsetAsync(counters + 3, 0, sizeof(int64_t), st));
  }

  if (r.thr > 0.0) {
    ReviveArgs ra{k, d, N, S, centroids, bias, chat, r.thr, seed, (uint64_t)t, flags, dead,
                  n0, rv_u, pair_i, pair_n, rv_pos, rv_head, rv_cbase, rv_clen, rv_heads,
                  rv_list, rv_nheads, counters, nullptr, 0, 1, sph ? 1 : 0};
    HIP_TRY(launch_revive(ra, st));
  }
  if (opts && opts->out_counts)
    HIP_TRY(hipMemcpyAsync(opts->out_counts, N, sizeof(float) * k, hipMemcpyDeviceToDevice, st));
  if (!(opts && opts->no_finalize) && last_pass_begun)
    HIP_TRY(launch_finalize(k, d, pass_counts, LS, centroids, sph, st));

  HIP_TRY(hipMemcpyAsync(host_stat, dstat, sizeof host_stat, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipMemcpyAsync(host_counters, counters, sizeof host_counters, hipMemcpyDeviceToHost, st));
  if (log_cap > 0)
    HIP_TRY(hipMemcpyAsync(opts->split_log, dlog, sizeof(int32_t) * 3 * (size_t)log_cap,
                           hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));

  if (stats) {
    fill_stats(r, stats);
    for (int e = 0; e < r.npass; ++e) {
      stats->obj[e] = r.rows[e] ? host_stat[e] / (double)r.rows[e] : 0.0;
      const double s2 = host_stat[EMEANS_MAX_PASSES + 2 * e], s1 = host_stat[EMEANS_MAX_PASSES + 2 * e + 1];
      stats->imbalance[e] = s1 > 0 ? (double)k * s2 / (s1 * s1) : 0.0;
      int64_t sp;
      memcpy(&sp, &host_stat[3 * EMEANS_MAX_PASSES + e], sizeof sp);
      stats->splits[e] = sp;
    }
    stats->n_splits = host_counters[0];
    stats->n_logged = host_counters[1] < log_cap ? host_counters[1] : log_cap;
    stats->dead_at_end = r.thr > 0.0 ? host_counters[2] : 0;
    if (profile) {
      double cls_ms[kClasses] = {};
      for (const Span& sp : spans) {
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, sp.a, sp.b) == hipSuccess) cls_ms[sp.cls] += ms;
      }
      stats->ms_assign = cls_ms[kAssign];
      stats->ms_bucket = cls_ms[kBucket];
      stats->ms_group = cls_ms[kGroup];
      stats->ms_update = cls_ms[kUpdate];
      stats->ms_revive = cls_ms[kRevive];
      stats->ms_sample = cls_ms[kSample];
    }
    stats->steps_run = t;
    stats->ms_total =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t_start).count();
  }

done:
  for (const Span& sp : spans) {
    (void)hipEventDestroy(sp.a);
    (void)hipEventDestroy(sp.b);
  }
  if (base) {
    const hipError_t e = hipFreeAsync(base, st);
    if (e != hipSuccess && rc == EMEANS_OK)
      rc = fail(EMEANS_EHIP, "hipFreeAsync: %s", hipGetErrorString(e));
    if (rc == EMEANS_OK) {
      const hipError_t e2 = hipStreamSynchronize(st);
      if (e2 != hipSuccess) rc = fail(EMEANS_EHIP, "hipStreamSynchronize: %s", hipGetErrorString(e2));
    }
  }
  return rc;
}

}  // extern "C"
