/*
 * emeans.h -- C ABI of the MI355X e-means library (libemeans.so).
 *
 * e-means is mini-batch k-means whose centroid statistics are exponential
 * moving averages (faiss contrib/e_means README, "How the centroid updates
 * work"): for each batch, every vector goes to its exact nearest centroid,
 * then for every cluster j
 *     N_j <- (1 - alpha) N_j + alpha n_j,   S_j <- (1 - alpha) S_j + alpha s_j,
 *     c_j  = S_j / N_j,
 * where n_j, s_j are the count and sum of the batch's vectors assigned to j.
 * B and alpha0 follow the README's scaling
 * laws ("Scaling laws", equations (1)-(3)); alpha decays along a cosine to
 * alpha0/10; clusters whose running count falls under a fraction of the mean
 * are revived every 5 batches by splitting a cluster drawn in proportion to
 * its size; at the end each centroid becomes the exact mean of the vectors
 * the last pass assigned to it (README "How the centroid updates work";
 * blog "k-means Reads Your Data 25 Times. Two Would Do.", section on the four
 * things e-means changes).
 *
 * Conventions for every entry point:
 *   - X, centroids, labels and dists are DEVICE pointers (HIP device memory on
 *     the current device), row-major and contiguous, owned by the caller. The
 *     library never copies data between host and device for the caller.
 *   - X is n x d, fp32, bf16, fp16, int8 codes, uint8 values or FP8 E4M3 codes
 *     (opts->dtype).
 *     Centroids are always k x d fp32 (for code data: in code space). Labels
 *     are int32 in [0, k). Distances are fp32 squared L2.
 *   - Work is queued on opts->stream (a hipStream_t; NULL = the null stream).
 *     emeans_train synchronises that stream before it returns (its statistics
 *     are host values); emeans_assign and emeans_batch_rows are asynchronous.
 *   - The library allocates its working memory stream-ordered on that stream
 *     and releases it before returning (emeans_train) or stream-ordered after
 *     the queued work (emeans_assign).
 *   - Return value: EMEANS_OK (0) or a negative emeans_status. On error,
 *     emeans_last_error() gives a message (thread-local). Arguments are checked
 *     before any work is queued; a failed HIP call returns EMEANS_EHIP.
 *   - Inputs are not checked for NaN or infinity (README "Data and centroids
 *     fit on 1 GPU"): such values give undefined labels, never a fault.
 */
#ifndef EMEANS_H
#define EMEANS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EMEANS_MAX_PASSES 64

/* EMEANS_I8: X holds int8 codes of the data (README "Data precision", INT8:
 * the caller encodes each dimension with a shift and a power-of-two scale,
 * code = clamp(rint((x - shift) * scale), -127, 127), and decodes the
 * centroids as c / scale + shift). Training runs in code space: running sums
 * and centroids are fp32 averages of the codes, and the nearest-centroid
 * search compares each row with the centroids rounded to int8 codes (nearest,
 * ties to even, clamped to [-127, 127]) exactly, in integers; the distances
 * are those of the codes. Requires d <= 43919 (the integer score then fits
 * int32) and no spherical mode. */
/* EMEANS_F8: X holds FP8 E4M3 codes (OCP E4M3: bias 7, subnormals, no
 * infinities, largest 448; README "Data precision", FP8) made up front by a
 * converter (emeans_fp8_encode: the nearest E4M3 value of (x - shift) *
 * scale, saturating at +-448). Training runs in code space as for int8; the
 * search compares each row with the centroids rounded to the nearest E4M3
 * value (ties to even, saturating), multiplying in FP8 and accumulating in
 * fp32, so labels are exact only up to fp32 rounding, as for fp32 data. No
 * spherical mode. */
/* EMEANS_F16: X holds IEEE binary16 values (README "Data precision", FP16:
 * data converted once by the caller). As for bf16 data, only the search is in
 * the 16-bit format: it compares each row with the centroids rounded to fp16
 * (nearest, ties to even, subnormals kept; magnitudes from 65520 up become
 * infinity, as the README's table of out-of-range values states), multiplying
 * in fp16 and accumulating in fp32. Running sums and centroids are fp32. */
/* EMEANS_U8: X holds uint8 values 0..255 (README "Data precision": INT8 and
 * UINT8 input numbers, e.g. raw descriptor bytes), used as they are. Running
 * sums and centroids are fp32 averages of the values; the search compares
 * each row exactly, in integers, with the centroids rounded to the nearest
 * uint8 (ties to even, clamped to [0, 255]), so labels and distances are
 * exact. Requires d <= 43919 and no spherical mode, as int8. */
enum emeans_dtype {
  EMEANS_F32 = 0,
  EMEANS_BF16 = 1,
  EMEANS_I8 = 2,
  EMEANS_F8 = 3,
  EMEANS_F16 = 4,
  EMEANS_U8 = 5
};

enum emeans_status {
  EMEANS_OK = 0,
  EMEANS_EINVAL = -1,     /* a size, pointer or option is out of range */
  EMEANS_EDTYPE = -2,     /* unsupported element type */
  EMEANS_ENOMEM = -3,     /* device allocation failed */
  EMEANS_EHIP = -4,       /* a HIP call or kernel launch failed */
  EMEANS_ENOTDEVICE = -5  /* a pointer is not device memory */
};

enum emeans_law { EMEANS_LAW_AUTO = 0, EMEANS_LAW_THROUGHPUT = 1, EMEANS_LAW_QUALITY = 2 };

/* Options. A zero-initialised struct (or a NULL pointer) means the defaults
 * of the README's "Settings" table. */
typedef struct emeans_opts {
  int32_t dtype;              /* emeans_dtype of X (default fp32) */
  int32_t batch_law;          /* emeans_law: auto = quality for d <= 16, else throughput */
  int64_t batch_size;         /* 0: from the batch law; > 0: this batch (capped at n),
                                 and alpha0 then follows equation (3) for it */
  double alpha0;              /* 0: equation (3), clamped to [1e-4, 1]; > 0: this value */
  double unused_threshold;    /* 0: default (0.1, or no revival when d <= 2);
                                 < 0: no revival; > 0: revive clusters whose running
                                 count is below this fraction of the mean count */
  int32_t no_finalize;        /* 0: last-pass exact means (default); 1: return the
                                 EMA centroids c = S / N */
  int32_t profile;            /* 1: time kernel classes with HIP events (stats->ms_*) */
  void* stream;               /* hipStream_t, NULL = null stream */
  /* Optional outputs for inspection and testing (NULL = not produced). */
  int32_t* trace_labels;      /* device, sum of all batch sizes: the label of every
                                 batch slot of every step, in step order */
  float* out_counts;          /* device, k: running counts N at the end */
  int32_t* split_log;         /* host, 3 * split_log_cap: (step, dead j, donor i) */
  int64_t split_log_cap;
  int64_t max_steps;          /* 0: all steps; > 0: stop after this many update steps
                                 (the schedule stays that of the full run); the
                                 closing mean is taken only if the last pass began */
  int32_t bf16_search;        /* 1: fp32 X is searched in bf16 (README "Data precision":
                                 the pages' GPU default): the rows and the centroids
                                 are rounded to bf16 (nearest, ties to even) for the
                                 nearest-centroid search only, and the distances are
                                 those of the rounded vectors; grouping, running sums
                                 and centroids use the fp32 rows. 0: fp32 X is searched
                                 in fp32 (exact). Ignored for X of other types. */
  int32_t spherical;          /* 1: spherical e-means (README "Spherical e-means"):
                                 each centroid is kept at norm 1 (S / N rescaled after
                                 every change; an all-zero centroid is left as is),
                                 a vector is assigned where its dot product is
                                 largest, the closing step rescales each cluster's
                                 mean to norm 1, and stats->obj is the mean of
                                 2 - 2 x similarity. Vectors are not normalised (nor
                                 checked): pass unit-norm rows for cosine semantics.
                                 emeans_assign: labels by the highest dot product with
                                 C as given, dists[i] = that similarity. fp32, bf16
                                 or fp16 X only (EINVAL with int8, uint8 or FP8 X). */
  int32_t lloyd;              /* 1: Lloyd iterations instead of e-means (the
                                 baseline of the blog's Lloyd section, Faiss's
                                 k-means, the loss e-means is timed against): each
                                 of the T passes (T a whole number) is one step over
                                 all n rows in row order with alpha = 1, so every
                                 centroid becomes the exact mean of its rows; after
                                 every pass but the last, the centroids left without
                                 a row are split off donors drawn in proportion to
                                 the row counts (the revival split, as Faiss
                                 refills empty clusters; no other revival). batch_size,
                                 alpha0 and unused_threshold are ignored; stats->obj
                                 holds the mean squared distance of every iteration's
                                 assignment. n < 2^31 (the 2^24 batch limit does not
                                 apply; a cluster of more than 2^24 rows divides by
                                 its fp32-rounded count). Not with emeans_begin. */
  double slow_ema;            /* kappa >= 1 (0: off): a second, slower EMA for unseen
                                 data (blog "k-means Reads Your Data 25 Times. Two
                                 Would Do.", section on what e-means changes; the
                                 pages give no decay, so this is a reading): when the
                                 last pass begins, a second pair (N', S') starts from
                                 (N, S) and each update of that pass applies the same
                                 recurrence to it with beta_t = fl32(alpha_t / kappa);
                                 a revival in that pass restarts both halves' pair
                                 from their split values. Requires slow_centroids;
                                 not with lloyd. kappa = 1 gives the EMA centroids. */
  float* slow_centroids;      /* device, k x d fp32 (with slow_ema): written by
                                 emeans_train / emeans_finalize with S' / N' (the
                                 EMA centroid where N' = 0, or everywhere if the last
                                 pass never began), rescaled to norm 1 in spherical
                                 mode; the closing mean is not applied to them */
  int32_t search;             /* fp32 X only: convert the rows on the fly, batch by
                                 batch, for the nearest-centroid search (README "Data
                                 precision", fp32 data converted batch by batch; the
                                 rows and the centroids become
                                 fmt((v - search_shift) * search_scale) in fp32):
                                 EMEANS_BF16 or EMEANS_F16 (the casts; a shift is
                                 the optional centering, scale 0 or 1) or EMEANS_F8
                                 (the FP8 converter: shift and scale from
                                 emeans_fp8_calibrate). Sums and centroids stay
                                 fp32 in data units, and distances and obj are
                                 given in data units (divided by scale^2).
                                 0: none, or bf16 when bf16_search is set (the same
                                 cast). Workspace B x d bytes (FP8) or 2 B x d. No
                                 centering or FP8 converter in spherical mode. */
  const float* search_shift;  /* device, d fp32, or NULL (0); owned by the caller and
                                 read until emeans_train returns, or until
                                 emeans_free for a model from emeans_begin */
  double search_scale;        /* EMEANS_F8: power of two in [2^-126, 2^126] */
} emeans_opts;

/* Recipe and statistics of a run (README "Settings and results": recipe, obj,
 * iteration_stats, n_splits). */
typedef struct emeans_stats {
  int64_t batch_size;
  int64_t total_steps;
  int64_t n_splits;                 /* dead clusters revived */
  int64_t n_logged;                 /* entries written to opts->split_log */
  int64_t dead_at_end;              /* clusters under the revival threshold at the end */
  double alpha0;
  double unused_threshold;          /* the threshold in effect (0 = no revival) */
  int32_t law;                      /* emeans_law actually used */
  int32_t n_passes;
  int64_t rows_per_pass[EMEANS_MAX_PASSES];
  int64_t steps_per_pass[EMEANS_MAX_PASSES];
  double obj[EMEANS_MAX_PASSES];       /* mean squared distance of the pass's vectors to
                                          the centroids they were assigned to, while
                                          the centroids move */
  double imbalance[EMEANS_MAX_PASSES]; /* k * sum n_j^2 / (sum n_j)^2 over the pass */
  int64_t splits[EMEANS_MAX_PASSES];   /* revivals during the pass */
  double ms_total;                     /* emeans_train wall clock */
  /* with opts->profile: summed device time of each kernel class, from HIP
     events recorded on opts->stream around the launches */
  double ms_assign, ms_bucket, ms_group, ms_update, ms_revive, ms_sample;
                                       /* ms_sample includes, with bf16_search, the
                                          gather and bf16 rounding of the batch rows */
  int64_t steps_run;                   /* update steps executed */
  /* with opts->profile: device time of each pass, from an event recorded on
     opts->stream before the pass's first launch to one after its statistics
     (0 for a pass that did not run); entries past n_passes are 0 */
  double pass_ms[EMEANS_MAX_PASSES];
} emeans_stats;

/* Scaling-law recipe for (n, d, k, T) and the given options; host only, no
 * device work (README "Scaling laws", "Parameters", "Manual overrides").
 * Fills batch_size, alpha0, law, unused_threshold, n_passes, rows_per_pass,
 * steps_per_pass and total_steps of *out. Errors: EINVAL if n < 1, d < 1,
 * k < 1, k > n, T <= 0, or more than EMEANS_MAX_PASSES passes. */
int emeans_recipe(int64_t n, int32_t d, int32_t k, double T, const emeans_opts* opts,
                  emeans_stats* out);

/* Train e-means for T passes (T may be fractional: the last pass then visits
 * floor(frac(T) * n) vectors) starting from k distinct rows of X chosen from
 * `seed`.
 *   X          device, n x d, opts->dtype
 *   centroids  device, k x d fp32, output (also the working centroids)
 *   labels     device, n int32, output or NULL: the label the final pass gave
 *              each row (README "Quick start"); -1 for rows that pass did
 *              not visit
 *   stats      host, output or NULL
 * Errors: EINVAL (sizes as for emeans_recipe, n >= 2^31, NULL X/centroids),
 * EDTYPE, ENOTDEVICE, ENOMEM, EHIP. Synchronises opts->stream. */
int emeans_train(const void* X, int64_t n, int32_t d, int32_t k, double T, uint64_t seed,
                 float* centroids, int32_t* labels, const emeans_opts* opts,
                 emeans_stats* stats);

/* Nearest centroid of each row of X (README "Settings and results":
 * em.assign): labels[i] = argmin_j ||x_i - c_j||^2 (lowest j on ties) and
 * dists[i] = that squared distance (fp32, >= 0). For bf16 X the centroids
 * are searched in bf16 (README "Data precision"); so are fp32 X and the
 * centroids with opts->bf16_search (rows and centroids rounded to bf16, the
 * distances those of the rounded vectors; workspace n x d bf16). For int8 X
 * the centroids (code space) are rounded to int8 codes and the labels and
 * distances are exact for the codes (see EMEANS_I8); likewise for uint8 X
 * with the centroids rounded to uint8 (EMEANS_U8). fp16 X is searched with
 * the centroids rounded to fp16 and FP8 X with them rounded to E4M3.
 *   X        device, n x d, opts->dtype      C       device, k x d fp32
 *   labels   device, n int32 output          dists   device, n fp32 output or NULL
 * Errors: EINVAL (n < 0, d < 1, k < 1, n >= 2^31, NULL pointers), EDTYPE,
 * ENOTDEVICE, ENOMEM, EHIP. Asynchronous on opts->stream. */
int emeans_assign(const void* X, int64_t n, int32_t d, const float* C, int32_t k,
                  int32_t* labels, float* dists, const emeans_opts* opts);

/* Nearest centroid of each row, as emeans_assign, with no memory allocation:
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). Arguments,
 * results and errors are those of emeans_assign. The working memory (the
 * centroid bias, the search copy of the centroids, and the converted rows
 * when opts->search or bf16_search converts fp32 rows) comes from one device
 * array of EMEANS_STATIC_SCRATCH_BYTES per GPU, held from the library's load
 * until the process ends. The need is 4k bytes, plus 2kd for a bf16/fp16
 * search copy or kd for int8/uint8/E4M3 codes, plus 2nd (nd for FP8) for
 * converted rows, each part rounded up to 256 bytes; sizes that need more
 * fail with EINVAL before any device work. Every call on one GPU uses the same array, so calls
 * that overlap on one GPU (on different streams, or from several threads
 * without ordering) race and give undefined results; calls queued on one
 * stream are ordered. Asynchronous on opts->stream. */
#define EMEANS_STATIC_SCRATCH_BYTES (32u << 20)
int emeans_assign_static(const void* X, int64_t n, int32_t d, const float* C, int32_t k,
                         int32_t* labels, float* dists, const emeans_opts* opts);

/* ---------------------------------------------------------------------------
 * Streaming training (README "Data too big for memory"): the loop that
 * emeans_train runs, fed batch by batch by the caller, for data that does not
 * fit on the device while the centroids do:
 *
 *   emeans_begin(n, d, k, T, seed, start, &opts, &m);   // recipe from (n, d, k, T)
 *   for each pass e (stats.rows_per_pass[e] rows, a fresh order):
 *     for each batch (exactly stats.batch_size rows, the last of a pass: the rest):
 *       emeans_accumulate(m, batch, rows, labels);    // once, or once per piece
 *       emeans_update(m);
 *     emeans_end_epoch(m);
 *   emeans_finalize(m, centroids, &stats);  emeans_free(m);
 *
 * The model checks the counts (rows per batch and per pass), not which rows
 * were sent. A batch too large for one call may be accumulated in pieces
 * followed by one update. Revival runs every fifth update; the closing mean
 * (each centroid the exact mean of the rows the last pass assigned to it) is
 * taken when every pass has ended. All work is queued on opts->stream.
 * ------------------------------------------------------------------------- */
typedef struct emeans_model emeans_model;

/* Start a run: the recipe of emeans_recipe(n, d, k, T, opts); start = device,
 * k x d fp32 starting centroids (copied; rescaled to norm 1 when
 * opts->spherical); seed drives the revival draws. opts->max_steps must be 0.
 * Errors: EINVAL (as emeans_recipe, n >= 2^31, NULL start or model), EDTYPE,
 * ENOTDEVICE, ENOMEM, EHIP. */
int emeans_begin(int64_t n, int32_t d, int32_t k, double T, uint64_t seed, const float* start,
                 const emeans_opts* opts, emeans_model** model);

/* Add `rows` rows (device, rows x d, opts->dtype of emeans_begin, row-major)
 * to the current batch: assignment with the current centroids, per-cluster
 * counts and sums. labels: device, rows int32 output (each row's label) or
 * NULL. Errors: EINVAL (NULL, rows < 1, more rows than the pass or the batch
 * has left, all passes ended), ENOTDEVICE, EHIP. */
int emeans_accumulate(emeans_model* m, const void* batch, int64_t rows, int32_t* labels);

/* One update step with the batch accumulated since the last update. Errors:
 * EINVAL (no rows, a batch other than the recipe's size that does not end
 * the pass, all steps run), EHIP. */
int emeans_update(emeans_model* m);

/* End the current pass. Errors: EINVAL (the pass did not visit exactly its
 * rows, rows accumulated without an update, all passes ended), EHIP. */
int emeans_end_epoch(emeans_model* m);

/* Centroids (device, k x d fp32 output): the closing mean when every pass has
 * ended (unless opts->no_finalize), else the current centroids; stats as for
 * emeans_train (host, or NULL). Synchronises the stream; the model stays
 * valid. Errors: EINVAL, ENOTDEVICE, EHIP. */
int emeans_finalize(emeans_model* m, float* centroids, emeans_stats* stats);

/* Closing mean from a second look at the rows (README "Several GPUs", the
 * paragraph on final_closing_mean, for callers who run their own batch loop):
 * once every pass has ended and before emeans_finalize, the caller may send
 * all rows once more, in any blocks of at most stats.batch_size rows, in one
 * fixed order.
 *   batch       device, rows x d, the dtype of emeans_begin
 *   labels      device, rows int32, or NULL. Given: the label the last pass
 *               gave each row (saved from emeans_accumulate); -1 marks a row
 *               that pass skipped, which is left out. NULL: each row is
 *               assigned once more to its nearest current centroid (the final
 *               EMA centroids, searched in the run's format) and counted there.
 *   labels_out  device, rows int32 output or NULL: the label each row was
 *               counted under (the given one, or the search's).
 * The first call discards the closing statistics the last pass gathered;
 * emeans_finalize then makes each centroid that received rows their exact
 * mean (rescaled to norm 1 in spherical mode) and keeps the EMA centroid of
 * every other cluster; with opts->no_finalize the replay has no effect. The
 * model keeps its EMA centroids throughout (emeans_finalize writes only the
 * caller's table), and the calls after an emeans_finalize start a new replay
 * from zero. A
 * given label outside [-1, k) is left out as well, and emeans_finalize then
 * fails with EINVAL. Errors: EINVAL (NULL model or batch, rows < 1 or above
 * the batch size, a pass still open), ENOTDEVICE, EHIP. Asynchronous on
 * opts->stream. */
int emeans_closing_add(emeans_model* m, const void* batch, int64_t rows, const int32_t* labels,
                       int32_t* labels_out);

/* Release the model and its device workspace (NULL is accepted). */
void emeans_free(emeans_model* m);

/* Rows visited by batch slots [start, start + count) of pass `pass` of a
 * training run with this seed (README "Data too big for memory": a fresh
 * order every pass, every vector once). pass = -1 gives the order whose first
 * k entries are the starting rows emeans_train takes for k clusters.
 * rows_out: device, count int32.
 * Errors: EINVAL (n < 1, n >= 2^31, pass < -1, start + count > n, NULL),
 * ENOTDEVICE, EHIP. Asynchronous on `stream`. */
int emeans_batch_rows(int64_t n, uint64_t seed, int32_t pass, int64_t start, int64_t count,
                      int32_t* rows_out, void* stream);

/* ---------------------------------------------------------------------------
 * int8 codes (README "Data precision", INT8: a per-dimension offset and a
 * single power-of-two factor, calibrated from a sample, map fp32 data to codes
 * that training and assignment take with opts->dtype = EMEANS_I8).
 * ------------------------------------------------------------------------- */

/* Calibrate from n sample rows (the caller picks the sample):
 * shift[j] = (min_j + max_j) / 2 over the sample's column j (fp64, stored
 * fp32); r = the largest |x - shift| over the sample (fp64); *scale = the
 * largest power of two s with s r <= 127 (1 when r = 0).
 *   X      device, n x d fp32     shift  device, d fp32 output
 *   scale  host, one double output
 * Errors: EINVAL (n < 1, n >= 2^31, d < 1, NULL), ENOTDEVICE, ENOMEM, EHIP.
 * Synchronises `stream`. */
int emeans_int8_calibrate(const float* X, int64_t n, int32_t d, float* shift, double* scale,
                          void* stream);

/* codes = clamp(rint((X - shift) * scale), -127, 127): the difference and the
 * product in fp32, rounding to nearest with ties to even; values beyond the
 * calibrated range go to the edge codes.
 *   X      device, n x d fp32     shift  device, d fp32
 *   scale  a power of two in [2^-126, 2^126]
 *   codes  device, n x d int8 output
 * Errors: EINVAL (n < 0, n >= 2^31, d < 1, scale not such a power of two,
 * NULL), ENOTDEVICE, EHIP. Asynchronous on `stream`. */
int emeans_int8_encode(const float* X, int64_t n, int32_t d, const float* shift, double scale,
                       int8_t* codes, void* stream);

/* Code-space vectors (centroids trained on codes) back to data space:
 * out = C / scale + shift in fp64, stored fp32.
 *   C      device, k x d fp32     shift  device, d fp32
 *   out    device, k x d fp32 output (may equal C)
 * Errors: EINVAL (k < 0, d < 1, scale as for emeans_int8_encode, NULL),
 * ENOTDEVICE, EHIP. Asynchronous on `stream`. */
int emeans_int8_decode(const float* C, int64_t k, int32_t d, const float* shift, double scale,
                       float* out, void* stream);

/* FP8 E4M3 codes: the same converter with the FP8 range. Calibration picks
 * the largest power of two s with s r <= 448; codes are the nearest E4M3
 * value of (x - shift) * s (difference and product in fp32), ties to the
 * even mantissa, saturating at +-448, as E4M3 bit patterns; decoding is as
 * for int8 (c / scale + shift in fp64). Arguments and errors as for the
 * int8 functions. */
int emeans_fp8_calibrate(const float* X, int64_t n, int32_t d, float* shift, double* scale,
                         void* stream);
int emeans_fp8_encode(const float* X, int64_t n, int32_t d, const float* shift, double scale,
                      uint8_t* codes, void* stream);
int emeans_fp8_decode(const float* C, int64_t k, int32_t d, const float* shift, double scale,
                      float* out, void* stream);

/* Message for the last non-zero return on this thread ("" if none). */
const char* emeans_last_error(void);

/* ABI version (major * 100 + minor). */
int emeans_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EMEANS_H */
