// Host-side launchers of the e-means kernels (internal to libemeans.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace emk {

// Assign: for batch slot r (row = rows ? rows[r] : r) of X, the nearest
// centroid by maximal score x.c - |c|^2/2 (equivalent to minimal squared
// distance). dt is the search type of X and `Cs`: 0 fp32 (Cs = C), 1 bf16
// (Cs = bf16 C-hat), 2 int8 (Cs = int8 codes q), 3 FP8 E4M3 (Cs = E4M3
// codes of C, products accumulated in fp32), 4 fp16 (Cs = fp16 C-hat), 5
// uint8 (Cs = the uint8 codes of C shifted by -128 as int8; the rows are
// shifted the same way inside the kernel, bias as for int8). `bias` = -|c|^2/2 computed
// from Cs as fp32, except for int8, where it holds -|q|^2 as int32 and the
// score is the exact integer 2 x.q - |q|^2. Writes labels[r], dists[r]
// (optional), counts[label] += 1 (optional) and obj[0] += sum of distances
// (optional). With `sim` (spherical e-means, bias = 0; fp32, bf16 or fp16)
// dists[r] is the similarity x.c and obj adds 2 - 2 x similarity.
hipError_t launch_assign(int dt, const void* X, int d, const uint32_t* rows, int nrows,
                         const void* Cs, const float* bias, int k, int32_t* labels, float* dists,
                         int32_t* counts, double* obj, bool sim, hipStream_t st);

// bf16 (f16 false) or fp16 data of dimension 32, 64, 96 or 128: points
// resident in registers, 32x32x16 MFMA tiles (same contract as launch_assign).
bool assign_bf16_resident_ok(int d, const void* X, const void* Chat);
hipError_t launch_assign_bf16_resident(const void* X, int d, const uint32_t* rows, int nrows,
                                       const void* Chat, const float* bias, int k,
                                       int32_t* labels, float* dists, int32_t* counts,
                                       double* obj, bool sim, bool f16, hipStream_t st);

// int8 codes (u8 false) or uint8 data of dimension 32 * KS <= 256: points
// resident in registers, 32x32x32 int8 MFMA tiles, exact integer scores
// (same contract as launch_assign with dt 2 or 5; bias holds -|q|^2 as int32).
bool assign_i8_resident_ok(int d, const void* X, const void* Cq);
hipError_t launch_assign_i8_resident(const void* X, int d, const uint32_t* rows, int nrows,
                                     const void* Cq, const float* bias, int k, int32_t* labels,
                                     float* dists, int32_t* counts, double* obj, bool u8,
                                     hipStream_t st);

// int8 codes (u8 false) or uint8 data of dimension 512 or 768: 64 points per
// wave resident in registers, centroid panels through a ring of direct
// global-to-LDS loads, 16x16x64 int8 MFMA tiles, exact integer scores (same
// contract as launch_assign with dt 2 or 5; bias holds -|q|^2 as int32).
bool assign_i8_wide_ok(int d, const void* X, const void* Cq);
hipError_t launch_assign_i8_wide(const void* X, int d, const uint32_t* rows, int nrows,
                                 const void* Cq, const float* bias, int k, int32_t* labels,
                                 float* dists, int32_t* counts, double* obj, bool u8,
                                 hipStream_t st);

// FP8 E4M3 codes of dimension 512 or 768: the same structure with 16x16x128
// FP8 MFMA tiles and fp32 scores (same contract as launch_assign with dt 3,
// which has no similarity mode; bias holds -|c|^2 / 2).
bool assign_f8_wide_ok(int d, const void* X, const void* Cf);
hipError_t launch_assign_f8_wide(const void* X, int d, const uint32_t* rows, int nrows,
                                 const void* Cf, const float* bias, int k, int32_t* labels,
                                 float* dists, int32_t* counts, double* obj, hipStream_t st);

// rows[r] = pi(start + r) for the keyed permutation pk.
hipError_t launch_sample_rows(const PermKey& pk, uint64_t start, int count, uint32_t* rows,
                              hipStream_t st);
hipError_t launch_sample_rows_i32(const PermKey& pk, uint64_t start, int count, int32_t* rows,
                                  hipStream_t st);

// C[j] = X[pi(j)] as fp32, j < k (rescaled to norm 1 when sph); dt is the
// data type of X: 0 fp32, 1 bf16, 2 int8, 3 FP8 E4M3, 4 fp16, 5 uint8.
hipError_t launch_init_centroids(int dt, const void* X, int d, const PermKey& pk, int k,
                                 float* C, bool sph, hipStream_t st);

// bias[j] = -|c_j|^2 / 2 in the search format (0 when sph). At most one
// search copy is non-null: Chat = bf16(C), or fp16(C) with chat_f16; Cq =
// int8 codes q of C (nearest, clamped to +-127; with cq_u8 the nearest uint8
// value, clamped to [0, 255], minus 128), and then bias[j] holds the int32
// -|q_j|^2 (the assign contract); Cf = E4M3 codes of C (nearest, saturating
// at +-448). Chat and Cf round (c - sshift) * sscale (sshift NULL: c * sscale),
// fp32 data converted on the fly; sshift = NULL and sscale = 1 otherwise.
hipError_t launch_prep(const float* C, int k, int d, float* bias, uint16_t* Chat, bool chat_f16,
                       int8_t* Cq, bool cq_u8, uint8_t* Cf, const float* sshift, float sscale,
                       bool sph, hipStream_t st);

// out[r] = fmt((X[rows[r]] - shift) * scale) for r < nrows (rows NULL: row r;
// shift NULL: 0), row-major: fmt 1 bf16 bits, 4 fp16 bits (both nearest, ties
// to even), 3 E4M3 codes (nearest, saturating at +-448).
hipError_t launch_convert_rows(const float* X, int d, const uint32_t* rows, int nrows, int fmt,
                               const float* shift, float scale, void* out, hipStream_t st);

// off = exclusive scan of counts (k+1 entries), cursor = off[0..k); ovf lists
// the grouping work items beyond the first R rows of each cluster as
// (cluster, part) pairs, *ovf_n of them (room for rows / R pairs). With acc:
// acc += counts, then counts = 0 (the counts of one piece of a batch join the
// update's totals). R must be a power of two (hipErrorInvalidValue otherwise).
hipError_t launch_scan(int32_t* counts, int k, int R, int32_t* off, int32_t* cursor,
                       int2* ovf, int32_t* ovf_n, int32_t* acc, hipStream_t st);

// Bucket the batch by label: pos = cursor[label]++, order[pos] = rows[r] (r
// when rows is NULL) and, when olab is non-null, olab[pos] = (that row,
// label); when
// out_labels is non-null also out_labels[rows[r]] = label. Rows whose label
// lies outside [0, k) are skipped.
hipError_t launch_scatter(const int32_t* labels, const uint32_t* rows, int nb, int k,
                          int32_t* cursor, uint32_t* order, int2* olab, int32_t* out_labels,
                          hipStream_t st);

// counts[labels[r]] += 1 for labels in [0, k); *bad += 1 for each label that is
// neither in [0, k) nor -1.
hipError_t launch_label_hist(const int32_t* labels, int nb, int k, int32_t* counts,
                             int32_t* bad, hipStream_t st);

// pass_counts += counts and LS += s_acc for every cluster with a count; counts
// and s_acc are reset.
hipError_t launch_closing_add(int k, int d, int32_t* counts, float* s_acc, int32_t* pass_counts,
                              float* LS, hipStream_t st);

// Rows per grouping work item (R of launch_scan and launch_group) for rows of
// d elements of type dt: 64, or more for rows of at most 1 KB.
int group_rows(int dt, int d);

// s_acc[j] += sum of X rows of cluster j (work items of at most R rows). A
// cluster held by one work item is stored, assuming s_acc[j] = 0, unless
// `add` (a later piece of the same update). olab (row ids and labels in
// bucketed order, from launch_scatter) may be NULL; with it, batches of small clusters
// of narrow rows are grouped by windows of the order.
hipError_t launch_group(int dt, const void* X, int d, const uint32_t* order,
                        const int2* olab, const int32_t* off, const int2* ovf,
                        const int32_t* ovf_n, int k, int R, int nb, float* s_acc, bool add,
                        hipStream_t st);

// EMA update of every cluster; resets counts and s_acc for the next step;
// pass_counts += counts; LS += s when LS is non-null; refreshes bias and the
// search format (Chat, Cq or Cf, at most one non-null; Chat and Cf of
// (c - sshift) * sscale as in launch_prep).
// sph: the centroids are rescaled to norm 1 and the bias is 0.
// N2 / S2 (slow pair, both or neither): the same recurrence with rate beta
// and 1 - beta = b2.
hipError_t launch_ema(int k, int d, float a, float b, int32_t* counts, float* s_acc, float* N,
                      float* S, float* C, float* bias, uint16_t* Chat, bool chat_f16, int8_t* Cq,
                      bool cq_u8, uint8_t* Cf, int32_t* pass_counts, float* LS, bool sph,
                      float beta, float b2, float* N2, float* S2, const float* sshift,
                      float sscale, hipStream_t st);

// a[i] *= f for i < n.
hipError_t launch_scale(float* a, int64_t n, float f, hipStream_t st);

// out[j] = S2[j] / N2[j] where N2[j] > 0, else C[j] (N2 NULL: out = C);
// rescaled to norm 1 with sph where N2[j] > 0.
hipError_t launch_slow_final(int k, int d, const float* N2, const float* S2, const float* C,
                             float* out, bool sph, hipStream_t st);

struct ReviveArgs {
  int k, d;
  float* N;
  float* S;
  float* C;
  float* bias;
  uint16_t* Chat;     // bf16 (fp16 with chat_f16) search copy of C, or NULL
  int8_t* Cq;         // int8 search codes of C (shifted uint8 codes with cq_u8), or NULL
  uint8_t* Cf;        // E4M3 search codes of C, or NULL
  double thr;
  uint64_t seed, step;
  // k-sized scratch
  int32_t* flags;     // 1 = under the threshold at this check
  int32_t* dead;      // dead clusters in index order (q-th dead = dead[q])
  float* n0;          // running counts at the check
  double* udraw;      // the q-th dead cluster's uniform draw
  int32_t* pair_i;    // donor of the q-th dead cluster
  float* pair_n;      // donor's count right after that split
  int32_t* pos;       // place of split q in its donor's chain
  int32_t* head_of;   // first split of a donor
  int32_t* cbase;     // start of a chain (indexed by its first split)
  int32_t* clen;      // length of a chain (indexed by its first split)
  int32_t* heads;     // first splits, compacted
  int32_t* list;      // splits grouped by chain, in chain order
  int32_t* nheads;    // [1]: number of chains
  int64_t* counters;  // [0] splits, [1] logged, [2] dead count, [3] splits this pass
  int32_t* log;       // 3 * log_cap
  int64_t log_cap;
  int count_only;
  int sph;            // spherical e-means: split centroids rescaled to norm 1, bias 0
  float* wlive;       // live counts (0 for dead) when k > 32768; k rounded up to 4096
  int chat_f16;       // Chat holds fp16 rather than bf16
  float* N2;          // slow pair (or NULL): a split copies both halves' N and S here
  float* S2;
  int cq_u8;          // Cq holds shifted uint8 codes
  const float* sshift;  // the search copy rounds (c - sshift) * sscale (launch_prep)
  float sscale;
  int empty_only;     // Lloyd: dead = clusters with no row (N < 0.5) instead of N < thr * mean
};
// Dead-cluster check and donor draws (one workgroup), then the splits of the
// running sums, one wave per donor chain.
hipError_t launch_revive(const ReviveArgs& a, hipStream_t st);

// sums[0] += sum n_j^2, sums[1] += sum n_j over pass_counts; zeroes them if `reset`.
hipError_t launch_pass_stats(int32_t* pass_counts, int k, double* sums, int reset, hipStream_t st);

// Rows of C rescaled to norm 1 (fp64 norm and quotient); zero rows stay zero.
hipError_t launch_normalize_rows(float* C, int k, int d, hipStream_t st);

// C[j] = LS[j] / pass_counts[j] where pass_counts[j] > 0 (rescaled to norm
// 1 when sph).
hipError_t launch_finalize(int k, int d, const int32_t* pass_counts, const float* LS, float* C,
                           bool sph, hipStream_t st);

// INT8 / FP8 codes (codes.hip). Calibration of shift (d fp32, device) and
// scale (one fp64, device: the largest power of two s with s r <= bound)
// from n sample rows; `work` holds calib_workspace_floats(n, d) floats
// (8-byte aligned).
size_t calib_workspace_floats(int64_t n, int d);
hipError_t launch_calibrate(const float* X, int64_t n, int d, float* shift, float* work,
                            double bound, double* scale, hipStream_t st);
// codes of (X - shift) * scale, n x d bytes: fmt 0 int8 (clamp(rint(.),
// -127, 127)), fmt 1 FP8 E4M3 (nearest, saturating at +-448).
hipError_t launch_encode(const float* X, int64_t n, int d, const float* shift, float scale,
                         int fmt, uint8_t* codes, hipStream_t st);
// out = C / scale + shift (fp64, stored fp32), k x d.
hipError_t launch_decode(const float* C, int64_t k, int d, const float* shift, double scale,
                         float* out, hipStream_t st);

}  // namespace emk
