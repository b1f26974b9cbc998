// C ABI of libemeans.so: argument checks, the scaling-law recipe, workspace
// and the stream-ordered step loop of e-means training.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <chrono>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "emeans.h"
#include "kernels.hpp"

using namespace emk;

// Device scratch of the allocation-free assignment (emeans_assign_static); host
// code reaches it only through the address hipGetSymbolAddress gives per device.
static __device__ __align__(256) unsigned char scratch[EMEANS_STATIC_SCRATCH_BYTES];

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

constexpr int kGroupRowsMin = 64;  // the smallest rows per grouping work item (group_rows)
constexpr int64_t kSampleRows = 1 << 20;  // sampled rows drawn per launch, at most
constexpr int kReviveEvery = 5;  // blog: dead clusters are checked every five batches

struct Recipe {
  int law = 0;
  bool lloyd = false;  // plain Lloyd iterations: B = n, alpha = 1, no revival
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
  if (o && o->lloyd) {
    // blog, Lloyd section: assign every vector, then move each centroid to the
    // exact mean of its vectors; T whole iterations
    if (T != floor(T) || T > EMEANS_MAX_PASSES)
      return fail(EMEANS_EINVAL, "lloyd mode needs a whole number of iterations 1..%d (got %g)",
                  EMEANS_MAX_PASSES, T);
    r.lloyd = true;
    r.law = o->batch_law ? o->batch_law : (d <= 16 ? EMEANS_LAW_QUALITY : EMEANS_LAW_THROUGHPUT);
    r.B = n;
    r.alpha0 = 1.0;
    r.thr = 0.0;
    r.npass = (int)T;
    r.S = 0;
    for (int e = 0; e < r.npass; ++e) {
      r.rows[e] = n;
      r.steps[e] = 1;
      r.S += 1;
    }
    return EMEANS_OK;
  }
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
  size_t total() const {
    size_t t = 0;
    for (auto& w : wants) t += (w.second + 255) & ~(size_t)255;
    return t == 0 ? 256 : t;
  }
  // Carve the buffers out of `base` (256-byte aligned, at least total() bytes).
  void place(void* base) {
    size_t off = 0;
    for (auto& w : wants) {
      *w.first = static_cast<char*>(base) + off;
      off += (w.second + 255) & ~(size_t)255;
    }
    used = total();
  }
  hipError_t alloc(void** base, hipStream_t st) {
    hipError_t e = hipMallocAsync(base, total(), st);
    if (e != hipSuccess) return e;
    place(*base);
    return hipSuccess;
  }
};

// Device scratch of the allocation-free assignment (emeans_assign_static):
// bias and search copies of the centroids, and the converted rows when a
// search converter is used. Every GPU the library runs on holds its own copy
// from the module's load until the process ends.
constexpr size_t kScratchBytes = EMEANS_STATIC_SCRATCH_BYTES;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once
// per device (the array's host-side name is not a device address).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(EMEANS_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(EMEANS_EINVAL, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(EMEANS_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return EMEANS_OK;
}

}  // namespace

// Checks of a training run that need no device: dtype, then the recipe's
// arguments and limits.
constexpr int32_t kMaxDimI8 = 43919;  // int8 search: |2 x.q| + |q|^2 < 2^31

// dtype supported; int8 codes and uint8 data: dimension limit and no
// spherical mode; FP8 codes: no spherical mode.
bool dtype_known(int32_t dtype) {
  return dtype == EMEANS_F32 || dtype == EMEANS_BF16 || dtype == EMEANS_I8 ||
         dtype == EMEANS_F8 || dtype == EMEANS_F16 || dtype == EMEANS_U8;
}

int check_dtype(int32_t d, const emeans_opts* opts) {
  const int32_t dtype = opts ? opts->dtype : EMEANS_F32;
  if (!dtype_known(dtype))
    return fail(EMEANS_EDTYPE,
                "dtype %d not supported (fp32 = 0, bf16 = 1, int8 = 2, fp8 = 3, fp16 = 4, "
                "uint8 = 5)", dtype);
  if ((dtype == EMEANS_I8 || dtype == EMEANS_U8) && d > kMaxDimI8)
    return fail(EMEANS_EINVAL, "int8 and uint8 data need d <= %d (got %d)", kMaxDimI8, d);
  if ((dtype == EMEANS_I8 || dtype == EMEANS_F8 || dtype == EMEANS_U8) && opts->spherical)
    return fail(EMEANS_EINVAL, "spherical e-means takes fp32, bf16 or fp16 data");
  return EMEANS_OK;
}

// A converter scale: a power of two that fp32 holds with room to spare.
bool pow2_scale(double s) {
  if (!(s >= 0x1p-126 && s <= 0x1p126)) return false;
  int e;
  return frexp(s, &e) == 0.5;
}

// The search format of fp32 data converted on the fly (README "Data
// precision", fp32 rows converted batch by batch): opts->search, or bf16 for
// bf16_search; 0 for other data types (bf16_search is ignored there).
int32_t search_format(const emeans_opts* opts) {
  if (!opts || opts->dtype != EMEANS_F32) return 0;
  if (opts->search) return opts->search;
  return opts->bf16_search ? EMEANS_BF16 : 0;
}

// The converter's options: a known format for fp32 data; the FP8 converter
// with its calibrated shift and power-of-two scale; the casts with an optional
// centering shift and scale 1; no centering or FP8 converter in spherical mode.
int check_search(const emeans_opts* opts) {
  if (!opts) return EMEANS_OK;
  const int32_t sf = opts->search;
  if (sf != 0 && sf != EMEANS_BF16 && sf != EMEANS_F16 && sf != EMEANS_F8)
    return fail(EMEANS_EINVAL, "search must be 0, bf16 (1), fp8 (3) or fp16 (4) (got %d)", sf);
  if (sf != 0 && opts->dtype != EMEANS_F32)
    return fail(EMEANS_EINVAL, "a search converter takes fp32 data");
  if (sf != 0 && opts->bf16_search && sf != EMEANS_BF16)
    return fail(EMEANS_EINVAL, "bf16_search conflicts with search = %d", sf);
  const int32_t f = search_format(opts);
  const double sc = opts->search_scale;
  if (f == 0) {
    if (opts->search_shift) return fail(EMEANS_EINVAL, "search_shift needs a search converter");
    if (!(sc == 0.0 || sc == 1.0))
      return fail(EMEANS_EINVAL, "search_scale needs the FP8 search converter");
    return EMEANS_OK;
  }
  if (f == EMEANS_F8) {
    if (!opts->search_shift)
      return fail(EMEANS_EINVAL, "the FP8 converter needs search_shift and search_scale "
                                 "(emeans_fp8_calibrate)");
    if (!pow2_scale(sc))
      return fail(EMEANS_EINVAL, "search_scale must be a power of two in [2^-126, 2^126] (got %g)",
                  sc);
  } else if (!(sc == 0.0 || sc == 1.0)) {
    return fail(EMEANS_EINVAL, "the bf16 and fp16 casts take search_scale 0 or 1 (got %g)", sc);
  }
  if (opts->spherical && (f == EMEANS_F8 || opts->search_shift))
    return fail(EMEANS_EINVAL, "spherical mode takes the plain bf16 and fp16 casts only "
                               "(no centering, no FP8 converter)");
  return EMEANS_OK;
}

// The slow EMA's options: kappa >= 1 with an output table, not in Lloyd mode.
int check_slow(const emeans_opts* opts) {
  if (!opts) return EMEANS_OK;
  const double kp = opts->slow_ema;
  if (!(kp == 0.0 || kp >= 1.0))
    return fail(EMEANS_EINVAL, "slow_ema must be 0 (off) or >= 1 (got %g)", kp);
  if (kp >= 1.0 && !opts->slow_centroids)
    return fail(EMEANS_EINVAL, "slow_ema needs slow_centroids");
  if (kp == 0.0 && opts->slow_centroids)
    return fail(EMEANS_EINVAL, "slow_centroids is set but slow_ema is 0");
  if (kp >= 1.0 && opts->lloyd) return fail(EMEANS_EINVAL, "slow_ema does not apply to lloyd");
  return EMEANS_OK;
}

int check_run_args(int64_t n, int32_t d, int32_t k, double T, const emeans_opts* opts) {
  int rc0 = check_dtype(d, opts);
  if (rc0) return rc0;
  if ((rc0 = check_slow(opts))) return rc0;
  if ((rc0 = check_search(opts))) return rc0;
  Recipe r;
  const int rc = make_recipe(n, d, k, T, opts, r);
  if (rc) return rc;
  if (n >= ((int64_t)1 << 31)) return fail(EMEANS_EINVAL, "n must be < 2^31");
  if (!r.lloyd && r.B >= ((int64_t)1 << 24))
    return fail(EMEANS_EINVAL, "batch size must be < 2^24 (counts are exact in fp32)");
  return EMEANS_OK;
}

// ---------------------------------------------------------------------------
// The training state of one e-means run: recipe, workspace (one stream-ordered
// allocation) and the step loop's position. emeans_train drives it with the
// on-device sampler; the streaming entry points (README "Data too big for
// memory") let the caller feed the batches.
// ---------------------------------------------------------------------------
#define HIP_RET(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess)                                                                  \
      return fail(e_ == hipErrorOutOfMemory ? EMEANS_ENOMEM : EMEANS_EHIP, "%s: %s (%s:%d)", \
                  #expr, hipGetErrorString(e_), __FILE__, __LINE__);                       \
  } while (0)

struct emeans_model {
  enum { kAssign = 0, kBucket, kGroup, kUpdate, kRevive, kSample, kClasses };
  struct Span {
    int cls;
    hipEvent_t a, b;
  };

  // configuration
  int64_t n = 0;
  int d = 0, k = 0;
  uint64_t seed = 0;
  Recipe r;
  hipStream_t st = nullptr;
  int dt = EMEANS_F32;  // emeans_dtype of X
  bool bf16 = false, i8 = false, u8 = false, f8 = false, f16 = false, sph = false,
       profile = false;
  // fp32 rows converted on the fly for the search (0: none; else the format,
  // 1 bf16, 4 fp16, 3 E4M3): fmt((x - sshift) * sscale) into xb each batch
  int32_t conv = 0;
  const float* sshift = nullptr;
  float sscale = 1.0f;
  bool hf = false;  // chat holds fp16 (fp16 data or the fp16 cast)
  bool no_finalize = false;
  double slow_k = 0.0;             // slow EMA: kappa (0 = off)
  float* slow_out = nullptr;       // caller's table for the slow centroids
  bool slow_started = false;       // the slow pair holds the last pass's statistics
  int32_t* trace = nullptr;
  float* out_counts = nullptr;
  int32_t* split_log = nullptr;
  int64_t log_cap = 0;
  std::chrono::steady_clock::time_point t_start;

  // position in the schedule
  int e = 0;              // current pass
  int64_t t = 0;          // update steps done
  int64_t rows_pass = 0;  // rows accumulated in the current pass
  int64_t rows_step = 0;  // rows accumulated since the last update
  int64_t trace_off = 0;
  bool last_begun = false;
  bool replay = false;    // the closing statistics come from emeans_closing_add

  // workspace
  void* base = nullptr;
  float* C = nullptr;  // working centroids (the caller's output buffer in emeans_train)
  uint32_t *rows = nullptr, *order = nullptr;
  int2* olab = nullptr;  // (row id, label) of each slot in bucketed order
  // steps whose sampled rows one launch produces (rows holds sample_steps
  // batches): a 65536-row launch keeps one wave per SIMD, each waiting on its
  // own Feistel chain, so the rows of up to 2^20 slots are drawn at once
  int64_t sample_steps = 1;
  int32_t *blab = nullptr, *pcounts = nullptr, *counts = nullptr, *cursor = nullptr,
          *off = nullptr, *ovf_n = nullptr, *pass_counts = nullptr, *flags = nullptr,
          *dead = nullptr, *dlog = nullptr, *pair_i = nullptr, *rv_pos = nullptr,
          *rv_head = nullptr, *rv_cbase = nullptr, *rv_clen = nullptr, *rv_heads = nullptr,
          *rv_list = nullptr, *rv_nheads = nullptr;
  double* rv_u = nullptr;
  int2* ovf = nullptr;
  float *s_acc = nullptr, *S = nullptr, *N = nullptr, *LS = nullptr, *bias = nullptr,
        *n0 = nullptr, *pair_n = nullptr, *wlive = nullptr;
  float *N2 = nullptr, *S2 = nullptr;  // slow pair (slow EMA)
  uint16_t* chat = nullptr;      // bf16 or fp16 search copy of C
  unsigned char* xb = nullptr;   // the batch rows converted for the search
  int8_t* cq = nullptr;   // int8 codes of C (int8 data; shifted uint8 codes for uint8 data)
  uint8_t* cf = nullptr;  // E4M3 codes of C (FP8 data)
  // per pass: [0, P) sum of distances, [P, 3P) sum n^2 and sum n, [3P, 4P) splits (int64)
  double* dstat = nullptr;
  int64_t* counters = nullptr;  // [0] splits, [1] logged, [2] dead count, [3] splits this pass
  int32_t* bad_labels = nullptr;  // labels outside [-1, k) sent to emeans_closing_add
  std::vector<Span> spans;
  // with profile: events around each pass (pass_a at its first launch, pass_b
  // after its statistics); pass_open while pass e's start is recorded
  hipEvent_t pass_a[EMEANS_MAX_PASSES] = {}, pass_b[EMEANS_MAX_PASSES] = {};
  bool pass_open = false;

  ~emeans_model() {
    for (const Span& sp : spans) {
      (void)hipEventDestroy(sp.a);
      (void)hipEventDestroy(sp.b);
    }
    for (int q = 0; q < EMEANS_MAX_PASSES; ++q) {
      if (pass_a[q]) (void)hipEventDestroy(pass_a[q]);
      if (pass_b[q]) (void)hipEventDestroy(pass_b[q]);
    }
    if (base) {
      (void)hipFreeAsync(base, st);
      (void)hipStreamSynchronize(st);
    }
  }

  // Device time of a kernel class: events recorded on the launch stream around it.
  template <typename F>
  hipError_t timed(int cls, F&& launch) {
    if (!profile) return launch();
    Span sp{cls, nullptr, nullptr};
    hipError_t er = hipEventCreate(&sp.a);
    if (er == hipSuccess) er = hipEventCreate(&sp.b);
    if (er != hipSuccess) return er;
    spans.push_back(sp);
    if ((er = hipEventRecord(sp.a, st)) != hipSuccess) return er;
    if ((er = launch()) != hipSuccess) return er;
    return hipEventRecord(sp.b, st);
  }

  // Start of pass e's device time (with profile; once per pass).
  hipError_t mark_pass_start() {
    if (!profile || pass_open || e >= EMEANS_MAX_PASSES) return hipSuccess;
    hipError_t er = hipEventCreate(&pass_a[e]);
    if (er == hipSuccess) er = hipEventCreate(&pass_b[e]);
    if (er == hipSuccess) er = hipEventRecord(pass_a[e], st);
    if (er == hipSuccess) pass_open = true;
    return er;
  }

  // Centroid table the search reads for rows of type dt.
  const void* search_table() const {
    return (i8 || u8) ? (const void*)cq
           : (f8 || conv == EMEANS_F8) ? (const void*)cf
           : chat ? (const void*)chat : (const void*)C;
  }

  ReviveArgs revive_args(bool count_only) {
    return ReviveArgs{k, d, N, S, C, bias, chat, cq, cf, r.thr, seed, (uint64_t)t, flags, dead, n0, rv_u,
                      pair_i, pair_n, rv_pos, rv_head, rv_cbase, rv_clen, rv_heads, rv_list,
                      rv_nheads, counters, count_only ? nullptr : dlog,
                      count_only ? 0 : log_cap, count_only ? 1 : 0, sph ? 1 : 0, wlive,
                      hf ? 1 : 0, slow_started ? N2 : nullptr, slow_started ? S2 : nullptr,
                      u8 ? 1 : 0, sshift, sscale, r.lloyd ? 1 : 0};
  }

  // Recipe, options and workspace; C = external (the caller's buffer) or own.
  int init(int64_t n_, int32_t d_, int32_t k_, double T, uint64_t seed_, const emeans_opts* opts,
           float* external_C) {
    t_start = std::chrono::steady_clock::now();
    n = n_;
    d = d_;
    k = k_;
    seed = seed_;
    const int32_t dtype = opts ? opts->dtype : EMEANS_F32;
    int rc = check_dtype(d, opts);
    if (rc) return rc;
    rc = make_recipe(n, d, k, T, opts, r);
    if (rc) return rc;
    if (n >= ((int64_t)1 << 31)) return fail(EMEANS_EINVAL, "n must be < 2^31");
    if (!r.lloyd && r.B >= ((int64_t)1 << 24))
      return fail(EMEANS_EINVAL, "batch size must be < 2^24 (counts are exact in fp32)");
    if (opts && opts->trace_labels && (rc = check_device(opts->trace_labels, "trace_labels")))
      return rc;
    if (opts && opts->out_counts && (rc = check_device(opts->out_counts, "out_counts"))) return rc;
    if ((rc = check_slow(opts))) return rc;
    if ((rc = check_search(opts))) return rc;
    if (opts && opts->search_shift && (rc = check_device(opts->search_shift, "search_shift")))
      return rc;
    if (opts && opts->slow_centroids &&
        (rc = check_device(opts->slow_centroids, "slow_centroids")))
      return rc;
    if (opts && opts->split_log && opts->split_log_cap < 0)
      return fail(EMEANS_EINVAL, "split_log_cap must be >= 0");
    st = static_cast<hipStream_t>(opts ? opts->stream : nullptr);
    dt = dtype;
    bf16 = dtype == EMEANS_BF16;
    conv = search_format(opts);  // fp32 rows converted into xb for the search
    sshift = conv ? opts->search_shift : nullptr;
    sscale = conv == EMEANS_F8 ? (float)opts->search_scale : 1.0f;
    i8 = dtype == EMEANS_I8;  // the search runs in int8 against cq
    u8 = dtype == EMEANS_U8;  // the same integer search on rows and codes shifted by -128
    f8 = dtype == EMEANS_F8;  // the search runs in FP8 against cf
    f16 = dtype == EMEANS_F16;  // the search runs in fp16 against chat
    hf = f16 || conv == EMEANS_F16;
    sph = opts && opts->spherical;
    profile = opts && opts->profile;
    no_finalize = opts && opts->no_finalize;
    trace = opts ? opts->trace_labels : nullptr;
    out_counts = opts ? opts->out_counts : nullptr;
    split_log = (opts && opts->split_log) ? opts->split_log : nullptr;
    log_cap = split_log ? opts->split_log_cap : 0;
    slow_k = opts ? opts->slow_ema : 0.0;
    slow_out = slow_k >= 1.0 ? opts->slow_centroids : nullptr;

    const size_t kd = (size_t)k * d;
    const int64_t B = r.B;
    Arena ar;
    if (!external_C) ar.want(&C, kd);
    sample_steps = r.lloyd ? 1 : (B < kSampleRows ? kSampleRows / B : 1);
    ar.want(&rows, r.lloyd ? (size_t)1 : (size_t)(B * sample_steps));
    ar.want(&order, (size_t)B);
    ar.want(&olab, (size_t)B);
    ar.want(&blab, (size_t)B);
    ar.want(&pcounts, (size_t)k);
    ar.want(&counts, (size_t)k);
    ar.want(&cursor, (size_t)k);
    ar.want(&off, (size_t)k + 1);
    ar.want(&ovf, (size_t)(B / kGroupRowsMin) + 1);
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
    if (k > 32768) ar.want(&wlive, (size_t)((k + 4095) / 4096) * 4096);
    ar.want(&s_acc, kd);
    ar.want(&S, kd);
    ar.want(&N, (size_t)k);
    ar.want(&LS, kd);
    if (slow_out) {
      ar.want(&N2, (size_t)k);
      ar.want(&S2, kd);
    }
    ar.want(&bias, (size_t)k);
    if (bf16 || f16 || conv == EMEANS_BF16 || conv == EMEANS_F16) ar.want(&chat, kd);
    if (i8 || u8) ar.want(&cq, kd);
    if (f8 || conv == EMEANS_F8) ar.want(&cf, kd);
    if (conv) ar.want(&xb, (size_t)B * d * (conv == EMEANS_F8 ? 1 : 2));
    ar.want(&dstat, (size_t)4 * EMEANS_MAX_PASSES);
    ar.want(&counters, 4);
  ar.want(&bad_labels, 1);
    if (log_cap > 0) ar.want(&dlog, (size_t)3 * log_cap);
    HIP_RET(ar.alloc(&base, st));
    if (external_C) C = external_C;
    // zero the statistics and every accumulator the step loop expects at zero
    HIP_RET(hipMemsetAsync(pcounts, 0, sizeof(int32_t) * k, st));
    HIP_RET(hipMemsetAsync(counts, 0, sizeof(int32_t) * k, st));
    HIP_RET(hipMemsetAsync(pass_counts, 0, sizeof(int32_t) * k, st));
    HIP_RET(hipMemsetAsync(s_acc, 0, sizeof(float) * kd, st));
    HIP_RET(hipMemsetAsync(S, 0, sizeof(float) * kd, st));
    HIP_RET(hipMemsetAsync(N, 0, sizeof(float) * k, st));
    HIP_RET(hipMemsetAsync(LS, 0, sizeof(float) * kd, st));
    HIP_RET(hipMemsetAsync(dstat, 0, sizeof(double) * 4 * EMEANS_MAX_PASSES, st));
    HIP_RET(hipMemsetAsync(counters, 0, sizeof(int64_t) * 4, st));
    HIP_RET(hipMemsetAsync(bad_labels, 0, sizeof(int32_t), st));
    return EMEANS_OK;
  }

  // Closing replay (README "Several GPUs", final_closing_mean): nb rows of X
  // in the caller's order with their last-pass labels (given; -1 = left out)
  // or, when given is NULL, labels from a search against the current (final
  // EMA) centroids. The first call replaces the closing statistics the last
  // pass gathered. labels_out, when non-null, receives the labels used.
  int closing_add(const void* X, int nb, const int32_t* given, int32_t* labels_out) {
    if (!replay) {
      HIP_RET(hipMemsetAsync(pass_counts, 0, sizeof(int32_t) * k, st));
      HIP_RET(hipMemsetAsync(LS, 0, sizeof(float) * (size_t)k * d, st));
      HIP_RET(hipMemsetAsync(bad_labels, 0, sizeof(int32_t), st));
      replay = true;
    }
    const int32_t* lab = given;
    if (given) {
      HIP_RET(launch_label_hist(given, nb, k, pcounts, bad_labels, st));
    } else {
      if (conv)
        HIP_RET(launch_convert_rows(static_cast<const float*>(X), d, nullptr, nb, conv, sshift,
                                    sscale, xb, st));
      HIP_RET(launch_assign(conv ? conv : dt, conv ? (const void*)xb : X, d, nullptr, nb,
                            search_table(), bias, k, blab, nullptr, pcounts, nullptr, sph, st));
      lab = blab;
    }
    if (labels_out)
      HIP_RET(hipMemcpyAsync(labels_out, lab, sizeof(int32_t) * nb, hipMemcpyDeviceToDevice, st));
    HIP_RET(launch_scan(pcounts, k, group_rows(dt, d), off, cursor, ovf, ovf_n, counts, st));
    HIP_RET(launch_scatter(lab, nullptr, nb, k, cursor, order, olab, nullptr, st));
    HIP_RET(launch_group(dt, X, d, order, olab, off, ovf, ovf_n, k, group_rows(dt, d), nb, s_acc, false,
                         st));
    HIP_RET(launch_closing_add(k, d, counts, s_acc, pass_counts, LS, st));
    return EMEANS_OK;
  }

  // One batch, or one piece of a batch, of nb rows (row = rows ? rows[r] : r
  // of X): assignment, bucketing by label, per-cluster sums into s_acc and the
  // counts of the update; out_labels[row] = label when non-null.
  int accumulate(const void* X, const uint32_t* rws, int nb, int32_t* out_labels) {
    if (nb <= 0) return EMEANS_OK;
    const bool add = rows_step > 0;
    if (conv)
      HIP_RET(timed(kSample, [&] {
        return launch_convert_rows(static_cast<const float*>(X), d, rws, nb, conv, sshift, sscale,
                                   xb, st);
      }));
    HIP_RET(timed(kAssign, [&] {
      if (conv)
        return launch_assign(conv, xb, d, nullptr, nb, search_table(), bias, k, blab, nullptr,
                             pcounts, dstat + e, sph, st);
      return launch_assign(dt, X, d, rws, nb, search_table(), bias, k, blab, nullptr, pcounts,
                           dstat + e, sph, st);
    }));
    if (trace) {
      HIP_RET(hipMemcpyAsync(trace + trace_off, blab, sizeof(int32_t) * nb,
                             hipMemcpyDeviceToDevice, st));
      trace_off += nb;
    }
    HIP_RET(timed(kBucket, [&] {
      hipError_t er = launch_scan(pcounts, k, group_rows(dt, d), off, cursor, ovf, ovf_n, counts,
                                  st);
      if (er != hipSuccess) return er;
      return launch_scatter(blab, rws, nb, k, cursor, order, olab, out_labels, st);
    }));
    HIP_RET(timed(kGroup, [&] {
      return launch_group(dt, X, d, order, olab, off, ovf, ovf_n, k, group_rows(dt, d), nb, s_acc, add,
                          st);
    }));
    rows_step += nb;
    rows_pass += nb;
    return EMEANS_OK;
  }

  // EMA update with what was accumulated since the last one; revival every
  // kReviveEvery updates.
  int update() {
    const float a = r.lloyd ? 1.0f : alpha_at(r.alpha0, t, r.S);
    const float b = 1.0f - a;
    const bool last = e == r.npass - 1;
    const bool slow = slow_out && last;
    if (slow && !slow_started) {  // the slow pair starts from the running pair
      HIP_RET(hipMemcpyAsync(N2, N, sizeof(float) * k, hipMemcpyDeviceToDevice, st));
      HIP_RET(hipMemcpyAsync(S2, S, sizeof(float) * (size_t)k * d, hipMemcpyDeviceToDevice, st));
      slow_started = true;
    }
    const float beta = slow ? (float)((double)a / slow_k) : 0.0f;
    const float b2 = 1.0f - beta;
    HIP_RET(timed(kUpdate, [&] {
      return launch_ema(k, d, a, b, counts, s_acc, N, S, C, bias, chat, hf, cq, u8, cf, pass_counts,
                        last ? LS : nullptr, sph, beta, b2, slow ? N2 : nullptr,
                        slow ? S2 : nullptr, sshift, sscale, st);
    }));
    // Lloyd: clusters left without a row are split off donors after every
    // update but the last (the last one's means are the result)
    if ((r.thr > 0.0 && (t + 1) % kReviveEvery == 0) || (r.lloyd && t + 1 < r.S)) {
      const ReviveArgs ra = revive_args(false);
      HIP_RET(timed(kRevive, [&] { return launch_revive(ra, st); }));
    }
    ++t;
    rows_step = 0;
    return EMEANS_OK;
  }

  // Pass statistics (imbalance, splits) of the current pass; next pass.
  int close_pass() {
    const bool last = e == r.npass - 1;
    HIP_RET(launch_pass_stats(pass_counts, k, dstat + EMEANS_MAX_PASSES + 2 * e, last ? 0 : 1, st));
    // per-pass split count: snapshot counters[3] then reset it
    HIP_RET(hipMemcpyAsync(dstat + 3 * EMEANS_MAX_PASSES + e, counters + 3, sizeof(int64_t),
                           hipMemcpyDeviceToDevice, st));
    HIP_RET(hipMemsetAsync(counters + 3, 0, sizeof(int64_t), st));
    if (pass_open) {
      HIP_RET(hipEventRecord(pass_b[e], st));
      pass_open = false;
    }
    ++e;
    rows_pass = 0;
    return EMEANS_OK;
  }

  // Dead count at the end, optional outputs, the closing mean when `closing`,
  // centroids into out_C (when it is not the working table), statistics.
  int finish(float* out_C, emeans_stats* stats, bool closing) {
    double host_stat[4 * EMEANS_MAX_PASSES];
    int64_t host_counters[4] = {0, 0, 0, 0};
    if (r.thr > 0.0 || r.lloyd) {
      const ReviveArgs ra = revive_args(true);
      HIP_RET(launch_revive(ra, st));
    }
    if (out_counts)
      HIP_RET(hipMemcpyAsync(out_counts, N, sizeof(float) * k, hipMemcpyDeviceToDevice, st));
    // the slow centroids come from the EMA centroids before the closing mean
    if (slow_out)
      HIP_RET(launch_slow_final(k, d, slow_started ? N2 : nullptr, S2, C, slow_out, sph, st));
    // the closing mean goes into the caller's table; the model's own working
    // centroids stay the EMA centroids (a later closing replay searches them)
    float* dst = out_C ? out_C : C;
    if (dst != C)
      HIP_RET(hipMemcpyAsync(dst, C, sizeof(float) * (size_t)k * d, hipMemcpyDeviceToDevice, st));
    if (closing) HIP_RET(launch_finalize(k, d, pass_counts, LS, dst, sph, st));
    HIP_RET(hipMemcpyAsync(host_stat, dstat, sizeof host_stat, hipMemcpyDeviceToHost, st));
    HIP_RET(hipMemcpyAsync(host_counters, counters, sizeof host_counters, hipMemcpyDeviceToHost, st));
    if (log_cap > 0)
      HIP_RET(hipMemcpyAsync(split_log, dlog, sizeof(int32_t) * 3 * (size_t)log_cap,
                             hipMemcpyDeviceToHost, st));
    int32_t host_bad = 0;
    if (replay)
      HIP_RET(hipMemcpyAsync(&host_bad, bad_labels, sizeof host_bad, hipMemcpyDeviceToHost, st));
    HIP_RET(hipStreamSynchronize(st));
    replay = false;  // the next emeans_closing_add starts a new replay
    if (host_bad)
      return fail(EMEANS_EINVAL,
                  "emeans_closing_add received %d labels outside [-1, k); those rows were left "
                  "out of the closing mean", host_bad);
    if (!stats) return EMEANS_OK;
    fill_stats(r, stats);
    for (int q = 0; q < r.npass; ++q) {
      // distances of converted rows are in converted units: back to data units
      const double u2 = (double)sscale * (double)sscale;
      stats->obj[q] = r.rows[q] ? host_stat[q] / (double)r.rows[q] / u2 : 0.0;
      const double s2 = host_stat[EMEANS_MAX_PASSES + 2 * q];
      const double s1 = host_stat[EMEANS_MAX_PASSES + 2 * q + 1];
      stats->imbalance[q] = s1 > 0 ? (double)k * s2 / (s1 * s1) : 0.0;
      int64_t sp;
      memcpy(&sp, &host_stat[3 * EMEANS_MAX_PASSES + q], sizeof sp);
      stats->splits[q] = sp;
    }
    stats->n_splits = host_counters[0];
    stats->n_logged = host_counters[1] < log_cap ? host_counters[1] : log_cap;
    stats->dead_at_end = (r.thr > 0.0 || r.lloyd) ? host_counters[2] : 0;
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
      for (int q = 0; q < EMEANS_MAX_PASSES; ++q) {
        float ms = 0.0f;
        stats->pass_ms[q] = (pass_a[q] && pass_b[q] && q < e &&
                             hipEventElapsedTime(&ms, pass_a[q], pass_b[q]) == hipSuccess)
                                ? ms
                                : 0.0;
      }
    }
    stats->steps_run = t;
    stats->ms_total =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t_start).count();
    return EMEANS_OK;
  }
};

extern "C" {

const char* emeans_last_error(void) { return g_err.c_str(); }

int emeans_version(void) { return 102; }

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
  if (pass < -1) return fail(EMEANS_EINVAL, "pass must be >= -1 (got %d)", pass);
  if (start < 0 || count < 0 || start + count > n)
    return fail(EMEANS_EINVAL, "slot range [%lld, %lld) outside [0, %lld)", (long long)start,
                (long long)(start + count), (long long)n);
  if (!rows_out) return fail(EMEANS_EINVAL, "rows_out is NULL");
  int rc = check_device(rows_out, "rows_out");
  if (rc) return rc;
  // pass -1: the order whose first k entries are emeans_train's starting rows
  const PermKey pk = pass < 0 ? make_perm_key((uint64_t)n, seed, kStreamInit, 0)
                              : make_perm_key((uint64_t)n, seed, kStreamPerm, (uint64_t)pass);
  const hipError_t e = launch_sample_rows_i32(pk, (uint64_t)start, (int)count, rows_out,
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EMEANS_EHIP, "sampler launch: %s", hipGetErrorString(e));
  return EMEANS_OK;
}

// emeans_assign and emeans_assign_static: the same checks and kernels; the
// workspace is allocated stream-ordered (use_scratch false) or carved out of
// the device array `scratch` (use_scratch true, nothing allocated).
static int assign_impl(const void* X, int64_t n, int32_t d, const float* C, int32_t k,
                       int32_t* labels, float* dists, const emeans_opts* opts, bool use_scratch) {
  g_err.clear();
  const int32_t dtype = opts ? opts->dtype : EMEANS_F32;
  if (!dtype_known(dtype))
    return fail(EMEANS_EDTYPE,
                "dtype %d not supported (fp32 = 0, bf16 = 1, int8 = 2, fp8 = 3, fp16 = 4, "
                "uint8 = 5)", dtype);
  if (n < 0 || n >= ((int64_t)1 << 31)) return fail(EMEANS_EINVAL, "n out of range (%lld)", (long long)n);
  if (d < 1) return fail(EMEANS_EINVAL, "d must be >= 1");
  if (k < 1) return fail(EMEANS_EINVAL, "k must be >= 1");
  if (!X || !C || !labels) return fail(EMEANS_EINVAL, "X, C and labels must not be NULL");
  int rc;
  if ((rc = check_dtype(d, opts))) return rc;
  if ((rc = check_search(opts))) return rc;
  const bool bf16 = dtype == EMEANS_BF16;
  const bool i8 = dtype == EMEANS_I8;
  const bool u8 = dtype == EMEANS_U8;
  const bool f8 = dtype == EMEANS_F8;
  const bool f16 = dtype == EMEANS_F16;
  const int32_t conv = search_format(opts);  // fp32 rows converted for the search
  void* base = nullptr;
  float* bias = nullptr;
  uint16_t* chat = nullptr;
  unsigned char* xb = nullptr;
  int8_t* cq = nullptr;
  uint8_t* cf = nullptr;
  Arena ar;
  ar.want(&bias, (size_t)k);
  if (bf16 || f16 || conv == EMEANS_BF16 || conv == EMEANS_F16) ar.want(&chat, (size_t)k * d);
  if (i8 || u8) ar.want(&cq, (size_t)k * d);
  if (f8 || conv == EMEANS_F8) ar.want(&cf, (size_t)k * d);
  if (conv) ar.want(&xb, (size_t)n * d * (conv == EMEANS_F8 ? 1 : 2));
  if (use_scratch && ar.total() > kScratchBytes)
    return fail(EMEANS_EINVAL,
                "emeans_assign_static needs %zu bytes of scratch for these sizes (at most %zu: "
                "centroid bias and search copy, plus the converted rows with a search "
                "converter)", ar.total(), kScratchBytes);
  if (n == 0) return EMEANS_OK;
  if ((rc = check_device(X, "X")) || (rc = check_device(C, "C")) ||
      (rc = check_device(labels, "labels")) || (dists && (rc = check_device(dists, "dists"))))
    return rc;
  hipStream_t st = static_cast<hipStream_t>(opts ? opts->stream : nullptr);
  if (opts && opts->search_shift && (rc = check_device(opts->search_shift, "search_shift")))
    return rc;
  const float* sshift = conv ? opts->search_shift : nullptr;
  const float sscale = conv == EMEANS_F8 ? (float)opts->search_scale : 1.0f;
  const bool hf = f16 || conv == EMEANS_F16;
  const bool sph = opts && opts->spherical;  // highest dot product, similarity out
  rc = EMEANS_OK;
  if (use_scratch) {
    void* sp = nullptr;
    if ((rc = scratch_address(&sp))) return rc;
    ar.place(sp);  // every buffer is written before it is read: nothing to clear
  } else {
    HIP_TRY(ar.alloc(&base, st));
  }
  HIP_TRY(launch_prep(C, k, d, bias, chat, hf, cq, u8, cf, sshift, sscale, sph, st));
  if (conv)
    HIP_TRY(launch_convert_rows(static_cast<const float*>(X), d, nullptr, (int)n, conv, sshift,
                                sscale, xb, st));
  {
    const int sdt = conv ? conv : dtype;
    const void* cs = (i8 || u8) ? (const void*)cq
                     : (f8 || conv == EMEANS_F8) ? (const void*)cf
                     : chat ? (const void*)chat : (const void*)C;
    HIP_TRY(launch_assign(sdt, conv ? (const void*)xb : X, d, nullptr, (int)n, cs, bias, k,
                          labels, dists, nullptr, nullptr, sph, st));
    // distances of converted rows are in converted units: back to data units
    if (dists && sscale != 1.0f)
      HIP_TRY(launch_scale(dists, n, (float)(1.0 / ((double)sscale * (double)sscale)), st));
  }
done:
  if (base) {
    const hipError_t e = hipFreeAsync(base, st);
    if (e != hipSuccess && rc == EMEANS_OK)
      rc = fail(EMEANS_EHIP, "hipFreeAsync: %s", hipGetErrorString(e));
  }
  return rc;
}

int emeans_assign(const void* X, int64_t n, int32_t d, const float* C, int32_t k,
                  int32_t* labels, float* dists, const emeans_opts* opts) {
  return assign_impl(X, n, d, C, k, labels, dists, opts, false);
}

int emeans_assign_static(const void* X, int64_t n, int32_t d, const float* C, int32_t k,
                         int32_t* labels, float* dists, const emeans_opts* opts) {
  return assign_impl(X, n, d, C, k, labels, dists, opts, true);
}

int emeans_train(const void* X, int64_t n, int32_t d, int32_t k, double T, uint64_t seed,
                 float* centroids, int32_t* labels, const emeans_opts* opts,
                 emeans_stats* stats) {
  g_err.clear();
  int rc;
  if ((rc = check_run_args(n, d, k, T, opts))) return rc;
  if (!X || !centroids) return fail(EMEANS_EINVAL, "X and centroids must not be NULL");
  if ((rc = check_device(X, "X")) || (rc = check_device(centroids, "centroids")) ||
      (labels && (rc = check_device(labels, "labels"))))
    return rc;
  const int64_t max_steps = opts ? opts->max_steps : 0;
  if (max_steps < 0) return fail(EMEANS_EINVAL, "max_steps must be >= 0");

  emeans_model m;
  if ((rc = m.init(n, d, k, T, seed, opts, centroids))) return rc;
  const Recipe& r = m.r;
  const int64_t B = r.B;
  const int64_t run_steps = (max_steps > 0 && max_steps < r.S) ? max_steps : r.S;
  hipStream_t st = m.st;
  if (labels) HIP_RET(hipMemsetAsync(labels, 0xFF, sizeof(int32_t) * (size_t)n, st));

  // starting centroids: k distinct rows (first k entries of the init permutation)
  HIP_RET(launch_init_centroids(m.dt, X, d, make_perm_key((uint64_t)n, seed, kStreamInit, 0), k,
                                m.C, m.sph, st));
  HIP_RET(launch_prep(m.C, k, d, m.bias, m.chat, m.hf, m.cq, m.u8, m.cf, m.sshift, m.sscale, m.sph,
                      st));

  for (int e = 0; e < r.npass && m.t < run_steps; ++e) {
    const bool last = e == r.npass - 1;
    m.last_begun = last;
    const PermKey pk = make_perm_key((uint64_t)n, seed, kStreamPerm, (uint64_t)e);
    HIP_RET(m.mark_pass_start());
    for (int64_t s = 0; s < r.steps[e] && m.t < run_steps; ++s) {
      const int64_t rem = r.rows[e] - s * B;
      const int nb = (int)(rem < B ? rem : B);
      // Lloyd iterations visit the rows in their own order (rows = NULL); the
      // sampler fills the rows of sample_steps steps at a time
      const int64_t g = s % m.sample_steps;
      if (!r.lloyd && g == 0) {
        const int64_t left = r.rows[e] - s * B;
        const int64_t cnt = left < B * m.sample_steps ? left : B * m.sample_steps;
        HIP_RET(m.timed(emeans_model::kSample, [&] {
          return launch_sample_rows(pk, (uint64_t)(s * B), (int)cnt, m.rows, st);
        }));
      }
      if ((rc = m.accumulate(X, r.lloyd ? nullptr : m.rows + g * B, nb,
                             (last && labels) ? labels : nullptr)))
        return rc;
      if ((rc = m.update())) return rc;
    }
    if ((rc = m.close_pass())) return rc;
  }
  return m.finish(centroids, stats, !m.no_finalize && m.last_begun);
}

int emeans_begin(int64_t n, int32_t d, int32_t k, double T, uint64_t seed, const float* start,
                 const emeans_opts* opts, emeans_model** model) {
  g_err.clear();
  int rc;
  if (!model) return fail(EMEANS_EINVAL, "model is NULL");
  *model = nullptr;
  if ((rc = check_run_args(n, d, k, T, opts))) return rc;
  if (opts && opts->lloyd) return fail(EMEANS_EINVAL, "lloyd is an emeans_train option");
  if (!start) return fail(EMEANS_EINVAL, "start must not be NULL");
  if ((rc = check_device(start, "start"))) return rc;
  if (opts && opts->max_steps) return fail(EMEANS_EINVAL, "max_steps is an emeans_train option");
  emeans_model* m = new (std::nothrow) emeans_model;
  if (!m) return fail(EMEANS_ENOMEM, "model allocation failed");
  rc = m->init(n, d, k, T, seed, opts, nullptr);
  if (rc == EMEANS_OK) {
    const hipError_t e1 =
        hipMemcpyAsync(m->C, start, sizeof(float) * (size_t)k * d, hipMemcpyDeviceToDevice, m->st);
    if (e1 != hipSuccess) rc = fail(EMEANS_EHIP, "copy of the starting centroids: %s", hipGetErrorString(e1));
  }
  if (rc == EMEANS_OK && m->sph) {  // spherical: the starting centroids rescaled to norm 1 too
    const hipError_t e3 = launch_normalize_rows(m->C, k, d, m->st);
    if (e3 != hipSuccess) rc = fail(EMEANS_EHIP, "normalise: %s", hipGetErrorString(e3));
  }
  if (rc == EMEANS_OK) {
    const hipError_t e2 =
        launch_prep(m->C, k, d, m->bias, m->chat, m->hf, m->cq, m->u8, m->cf, m->sshift, m->sscale,
                    m->sph, m->st);
    if (e2 != hipSuccess) rc = fail(EMEANS_EHIP, "centroid prep: %s", hipGetErrorString(e2));
  }
  if (rc != EMEANS_OK) {
    delete m;
    return rc;
  }
  *model = m;
  return EMEANS_OK;
}

int emeans_accumulate(emeans_model* m, const void* batch, int64_t rows, int32_t* labels) {
  g_err.clear();
  int rc;
  if (!m) return fail(EMEANS_EINVAL, "model is NULL");
  if (!batch) return fail(EMEANS_EINVAL, "batch is NULL");
  if (rows < 1) return fail(EMEANS_EINVAL, "rows must be >= 1 (got %lld)", (long long)rows);
  if (m->e >= m->r.npass)
    return fail(EMEANS_EINVAL, "all %d passes of the recipe have ended", m->r.npass);
  if (m->rows_pass + rows > m->r.rows[m->e])
    return fail(EMEANS_EINVAL, "pass %d visits %lld rows: %lld more would exceed it", m->e,
                (long long)m->r.rows[m->e], (long long)rows);
  if (m->rows_step + rows > m->r.B)
    return fail(EMEANS_EINVAL, "a batch has at most %lld rows (the recipe's batch size)",
                (long long)m->r.B);
  if ((rc = check_device(batch, "batch")) || (labels && (rc = check_device(labels, "labels"))))
    return rc;
  if (m->e == m->r.npass - 1) m->last_begun = true;
  HIP_RET(m->mark_pass_start());
  return m->accumulate(batch, nullptr, (int)rows, labels);
}

int emeans_update(emeans_model* m) {
  g_err.clear();
  if (!m) return fail(EMEANS_EINVAL, "model is NULL");
  if (m->rows_step < 1) return fail(EMEANS_EINVAL, "no rows accumulated since the last update");
  if (m->rows_step != m->r.B && m->rows_pass != m->r.rows[m->e])
    return fail(EMEANS_EINVAL,
                "a batch must have exactly %lld rows except the last of a pass (got %lld)",
                (long long)m->r.B, (long long)m->rows_step);
  if (m->t >= m->r.S) return fail(EMEANS_EINVAL, "all %lld update steps have run", (long long)m->r.S);
  return m->update();
}

int emeans_end_epoch(emeans_model* m) {
  g_err.clear();
  if (!m) return fail(EMEANS_EINVAL, "model is NULL");
  if (m->e >= m->r.npass) return fail(EMEANS_EINVAL, "all %d passes have ended", m->r.npass);
  if (m->rows_step) return fail(EMEANS_EINVAL, "rows accumulated without an update");
  if (m->rows_pass != m->r.rows[m->e])
    return fail(EMEANS_EINVAL, "pass %d must visit %lld rows (got %lld)", m->e,
                (long long)m->r.rows[m->e], (long long)m->rows_pass);
  return m->close_pass();
}

int emeans_finalize(emeans_model* m, float* centroids, emeans_stats* stats) {
  g_err.clear();
  int rc;
  if (!m) return fail(EMEANS_EINVAL, "model is NULL");
  if (!centroids) return fail(EMEANS_EINVAL, "centroids must not be NULL");
  if ((rc = check_device(centroids, "centroids"))) return rc;
  return m->finish(centroids, stats, !m->no_finalize && m->e == m->r.npass);
}

int emeans_closing_add(emeans_model* m, const void* batch, int64_t rows, const int32_t* labels,
                       int32_t* labels_out) {
  g_err.clear();
  int rc;
  if (!m) return fail(EMEANS_EINVAL, "model is NULL");
  if (!batch) return fail(EMEANS_EINVAL, "batch is NULL");
  if (m->e < m->r.npass)
    return fail(EMEANS_EINVAL, "the closing replay starts after the last pass has ended "
                "(pass %d of %d is open)", m->e, m->r.npass);
  if (rows < 1 || rows > m->r.B)
    return fail(EMEANS_EINVAL, "rows must be in [1, %lld] (the batch size), got %lld",
                (long long)m->r.B, (long long)rows);
  if ((rc = check_device(batch, "batch")) || (labels && (rc = check_device(labels, "labels"))) ||
      (labels_out && (rc = check_device(labels_out, "labels_out"))))
    return rc;
  return m->closing_add(batch, (int)rows, labels, labels_out);
}

void emeans_free(emeans_model* m) { delete m; }

// README "Data precision", INT8: calibration, encoding and decoding of codes.

namespace {

int calibrate_codes(const float* X, int64_t n, int32_t d, float* shift, double* scale,
                    double bound, void* stream) {
  if (n < 1 || n >= ((int64_t)1 << 31)) return fail(EMEANS_EINVAL, "n out of range (%lld)", (long long)n);
  if (d < 1) return fail(EMEANS_EINVAL, "d must be >= 1");
  if (!X || !shift || !scale) return fail(EMEANS_EINVAL, "X, shift and scale must not be NULL");
  int rc;
  if ((rc = check_device(X, "X")) || (rc = check_device(shift, "shift"))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* base = nullptr;
  float* work = nullptr;
  double* dscale = nullptr;
  Arena ar;
  ar.want(&dscale, 1);
  ar.want(&work, calib_workspace_floats(n, d));
  rc = EMEANS_OK;
  HIP_TRY(ar.alloc(&base, st));
  HIP_TRY(launch_calibrate(X, n, d, shift, work, bound, dscale, st));
  HIP_TRY(hipMemcpyAsync(scale, dscale, sizeof(double), hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
done:
  if (base) {
    const hipError_t e = hipFreeAsync(base, st);
    if (e != hipSuccess && rc == EMEANS_OK)
      rc = fail(EMEANS_EHIP, "hipFreeAsync: %s", hipGetErrorString(e));
  }
  return rc;
}

int encode_codes(const float* X, int64_t n, int32_t d, const float* shift, double scale, int fmt,
                 uint8_t* codes, void* stream) {
  if (n < 0 || n >= ((int64_t)1 << 31)) return fail(EMEANS_EINVAL, "n out of range (%lld)", (long long)n);
  if (d < 1) return fail(EMEANS_EINVAL, "d must be >= 1");
  if (!pow2_scale(scale)) return fail(EMEANS_EINVAL, "scale must be a power of two in [2^-126, 2^126] (got %g)", scale);
  if (!X || !shift || !codes) return fail(EMEANS_EINVAL, "X, shift and codes must not be NULL");
  if (n == 0) return EMEANS_OK;
  int rc;
  if ((rc = check_device(X, "X")) || (rc = check_device(shift, "shift")) ||
      (rc = check_device(codes, "codes")))
    return rc;
  const hipError_t e =
      launch_encode(X, n, d, shift, (float)scale, fmt, codes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EMEANS_EHIP, "encode launch: %s", hipGetErrorString(e));
  return EMEANS_OK;
}

}  // namespace

int emeans_int8_calibrate(const float* X, int64_t n, int32_t d, float* shift, double* scale,
                          void* stream) {
  g_err.clear();
  return calibrate_codes(X, n, d, shift, scale, 127.0, stream);
}

int emeans_int8_encode(const float* X, int64_t n, int32_t d, const float* shift, double scale,
                       int8_t* codes, void* stream) {
  g_err.clear();
  return encode_codes(X, n, d, shift, scale, 0, reinterpret_cast<uint8_t*>(codes), stream);
}

int emeans_int8_decode(const float* C, int64_t k, int32_t d, const float* shift, double scale,
                       float* out, void* stream) {
  g_err.clear();
  if (k < 0 || k >= ((int64_t)1 << 31)) return fail(EMEANS_EINVAL, "k out of range (%lld)", (long long)k);
  if (d < 1) return fail(EMEANS_EINVAL, "d must be >= 1");
  if (!pow2_scale(scale)) return fail(EMEANS_EINVAL, "scale must be a power of two in [2^-126, 2^126] (got %g)", scale);
  if (!C || !shift || !out) return fail(EMEANS_EINVAL, "C, shift and out must not be NULL");
  if (k == 0) return EMEANS_OK;
  int rc;
  if ((rc = check_device(C, "C")) || (rc = check_device(shift, "shift")) ||
      (rc = check_device(out, "out")))
    return rc;
  const hipError_t e = launch_decode(C, k, d, shift, scale, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EMEANS_EHIP, "decode launch: %s", hipGetErrorString(e));
  return EMEANS_OK;
}

int emeans_fp8_calibrate(const float* X, int64_t n, int32_t d, float* shift, double* scale,
                         void* stream) {
  g_err.clear();
  return calibrate_codes(X, n, d, shift, scale, 448.0, stream);
}

int emeans_fp8_encode(const float* X, int64_t n, int32_t d, const float* shift, double scale,
                      uint8_t* codes, void* stream) {
  g_err.clear();
  return encode_codes(X, n, d, shift, scale, 1, codes, stream);
}

int emeans_fp8_decode(const float* C, int64_t k, int32_t d, const float* shift, double scale,
                      float* out, void* stream) {
  return emeans_int8_decode(C, k, d, shift, scale, out, stream);
}

}  // extern "C"
