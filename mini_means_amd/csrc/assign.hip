// Fused nearest-centroid assignment for gfx950 (MFMA, wave64).
//
// A workgroup of 8 waves owns a tile of 128 points and sweeps every centroid
// in panels of 256. For each (panel, d-chunk) the point rows and centroid
// rows are staged through LDS (double buffered, one 128-byte slab per row);
// each wave computes a 64 x 64 block of scores with 16x16 MFMA tiles:
//   fp32 X: v_mfma_f32_16x16x4_f32     bf16 X: v_mfma_f32_16x16x32_bf16
//   int8 X: v_mfma_i32_16x16x64_i8     FP8 E4M3 X: v_mfma_f32_16x16x32_fp8_fp8
//   fp16 X: v_mfma_f32_16x16x32_f16.
// The stage ring (16-byte aligned rows) takes FP8 through the gfx950
// v_mfma_scale_f32_16x16x128_f8f6f4 (scales 1) instead: one instruction per
// 128-byte stage, each lane holding its 16-byte piece of both 64-byte slices.
// Centroids sit on the MFMA M dimension and points on N, so after a tile each
// lane holds four centroid scores of a single point; the running best score
// and its index stay in registers across all panels and are merged across the
// four lane groups with cross-lane shuffles and across the four M-waves
// through LDS only once at the end. The score is x.c - |c|^2/2: the bias
// -|c|^2/2 is the accumulator's initial value, so the argmax needs compares
// only, and the squared distance is |x|^2 - 2 * best. No n x k distance
// matrix is formed. A 256-centroid panel means the gathered point rows, the
// data least likely to sit in L2, are re-read k/256 times per batch.
//
// Ties: each lane visits its centroids in increasing index order and keeps
// the first strict maximum; merges prefer the lower index on equal scores, so
// the lowest index wins overall, matching argmin over the squared distance.
//
// int8 codes against int8 centroid codes q: the products accumulate exactly
// in int32 from zero and the score is the integer 2 x.q - |q|^2 (the bias
// array then holds -|q|^2 as int32), so labels and distances are exact.
// With d <= 43919 no intermediate leaves the int32 range:
// |2 x.q| + |q|^2 <= d (2 * 128 * 127 + 127^2) < 2^31.
//
// uint8 rows run the same integer search after a shift by -128 (u ^ 0x80
// read as int8 is u - 128), applied to the point chunks as they leave LDS or
// memory; the centroids' codes are stored already shifted. Distances are
// unchanged by the shift, and per dimension the score 2 x'q' - q'^2 lies in
// [-48896, 16384], so d <= 43919 keeps the sum inside int32 here too.
#include "kernels.hpp"

namespace emk {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Per data type (0 fp32, 1 bf16, 2 int8, 3 FP8 E4M3, 4 fp16, 5 uint8):
// element bytes, the accumulator tile and the score type.
template <int DT>
struct Fmt {
  static constexpr int ES = 4;
  using Acc = f32x4;
  using Sc = float;
};
template <>
struct Fmt<1> {
  static constexpr int ES = 2;
  using Acc = f32x4;
  using Sc = float;
};
template <>
struct Fmt<2> {
  static constexpr int ES = 1;
  using Acc = i32x4;
  using Sc = int;
};
template <>
struct Fmt<3> {
  static constexpr int ES = 1;
  using Acc = f32x4;
  using Sc = float;
};
template <>
struct Fmt<5> : Fmt<2> {};
template <>
struct Fmt<4> {
  static constexpr int ES = 2;
  using Acc = f32x4;
  using Sc = float;
};

// int8 and uint8 rows: the exact integer search
template <int DT>
constexpr bool kIntSearch = DT == 2 || DT == 5;

// A 16-byte chunk of point data in the search's form: uint8 bytes shifted
// by -128 into int8 (the centroid codes are stored shifted already).
template <int DT>
__device__ __forceinline__ u32x4 point_chunk(u32x4 w) {
  if constexpr (DT == 5) return w ^ 0x80808080u;
  return w;
}

constexpr int kWM = 4;               // waves along the centroid (M) dimension
constexpr int kWN = 2;               // waves along the point (N) dimension
constexpr int kTP = 64 * kWN;        // points per workgroup
constexpr int kTC = 64 * kWM;        // centroids per panel
constexpr int kThreads = 64 * kWM * kWN;
constexpr int kSlab = 128;           // bytes of one row per stage
constexpr int kStride = 144;         // LDS row pitch in bytes (slab + 16 to spread banks)
constexpr int kChunks = kSlab / 16;  // 16-byte chunks per row slab
constexpr int kRowsPerPass = kThreads / kChunks;
constexpr int kXL = kTP / kRowsPerPass;     // point-row slabs per thread
constexpr int kCL = kTC / kRowsPerPass;     // centroid-row slabs per thread

template <int DT, bool VEC>
__device__ __forceinline__ u32x4 load_slab16(const unsigned char* row, int col, int d) {
  // 16 bytes of a row starting at element `col`. With whole 16-byte chunks
  // per row (VEC) the address is clamped into the row and the caller zeroes
  // chunks past the end when it stores them, so the load stays in flight
  // across the MFMA work; otherwise elements past the end read as zero (as
  // 0x80 for uint8 rows, which point_chunk maps to zero).
  constexpr int ES = Fmt<DT>::ES;
  constexpr int EPV = 16 / ES;
  if constexpr (VEC) {
    return *reinterpret_cast<const u32x4*>(row + (size_t)(col < d ? col : d - EPV) * ES);
  } else {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const int c = col + e;
      uint32_t v = DT == 5 ? 0x80u : 0u;
      if (c < d) {
        if constexpr (ES == 1)
          v = (uint32_t)row[c];
        else if constexpr (ES == 2)
          v = (uint32_t)reinterpret_cast<const uint16_t*>(row)[c];
        else
          v = reinterpret_cast<const uint32_t*>(row)[c];
      }
      constexpr int PW = 4 / ES;  // elements per 32-bit word
      w[e / PW] |= v << (8 * ES * (e % PW));
    }
    return u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Sum of squares of the elements in a 16-byte chunk (exact integer for int8;
// uint8 chunks arrive shifted into int8 by point_chunk).
template <int DT>
__device__ __forceinline__ typename Fmt<DT>::Sc sumsq16(u32x4 w) {
  typename Fmt<DT>::Sc s = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (kIntSearch<DT>) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int v = (int)(int8_t)(w[e] >> (8 * b));
        s += v * v;
      }
    } else if constexpr (DT == 3) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float v = e4m3_to_f32((w[e] >> (8 * b)) & 0xFFu);
        s += v * v;
      }
    } else if constexpr (DT == 1) {
      const float lo = __uint_as_float(w[e] << 16);
      const float hi = __uint_as_float(w[e] & 0xFFFF0000u);
      s += lo * lo + hi * hi;
    } else if constexpr (DT == 4) {
      const float lo = f16_to_f32((uint16_t)(w[e] & 0xFFFFu));
      const float hi = f16_to_f32((uint16_t)(w[e] >> 16));
      s += lo * lo + hi * hi;
    } else {
      const float f = __uint_as_float(w[e]);
      s += f * f;
    }
  }
  return s;
}

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// FP8 E4M3: both 64-byte slices of a 128-byte stage for a 64 x 64 score block
// (a[s][mb], b[s][nb]: slice s, 16 bytes per lane, lane / 16 selecting the
// piece), one 16x16x128 MFMA per tile. A and B pair the same bytes with the
// same lanes, so every product meets its partner.
__device__ __forceinline__ void mfma_stage_f8(f32x4 (&acc)[4][4], const u32x4 (&a)[2][4],
                                              const u32x4 (&b)[2][4]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const i32x8 av = {(int)a[0][mb][0], (int)a[0][mb][1], (int)a[0][mb][2], (int)a[0][mb][3],
                        (int)a[1][mb][0], (int)a[1][mb][1], (int)a[1][mb][2], (int)a[1][mb][3]};
      const i32x8 bv = {(int)b[0][nb][0], (int)b[0][nb][1], (int)b[0][nb][2], (int)b[0][nb][3],
                        (int)b[1][nb][0], (int)b[1][nb][1], (int)b[1][nb][2], (int)b[1][nb][3]};
      // formats 0, 0: E4M3 operands; scales 127: 2^0
      acc[mb][nb] =
          __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[mb][nb], 0, 0, 0, 127, 0, 127);
    }
}

// One 64-byte slice of K for a 64 x 64 score block: a[mb] holds 16 centroid
// rows, b[nb] 16 point rows, 16 bytes per lane (lane / 16 selects the 16-byte
// piece of the slice).
template <int DT>
__device__ __forceinline__ void mfma_slice(typename Fmt<DT>::Acc (&acc)[4][4], const u32x4 (&a)[4],
                                           const u32x4 (&b)[4]) {
  if constexpr (kIntSearch<DT>) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a[mb]),
                                                            __builtin_bit_cast(i32x4, b[nb]),
                                                            acc[mb][nb], 0, 0, 0);
  } else if constexpr (DT == 3) {
    // two K = 32 steps: the low and the high 8 bytes of each lane's chunk
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const long av = (long)(((uint64_t)a[mb][2 * h + 1] << 32) | a[mb][2 * h]);
          const long bv = (long)(((uint64_t)b[nb][2 * h + 1] << 32) | b[nb][2 * h]);
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(av, bv, acc[mb][nb], 0, 0, 0);
        }
  } else if constexpr (DT == 1) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a[mb]), __builtin_bit_cast(bf16x8, b[nb]), acc[mb][nb], 0,
            0, 0);
  } else if constexpr (DT == 4) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[mb]),
                                                             __builtin_bit_cast(f16x8, b[nb]),
                                                             acc[mb][nb], 0, 0, 0);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
              __uint_as_float(a[mb][q]), __uint_as_float(b[nb][q]), acc[mb][nb], 0, 0, 0);
  }
}

// Part [P0, P1) of mfma_slice: fp32 k-steps P0..P1-1 of the slice (each
// lane's chunk holds four consecutive k values); other types the MFMAs of
// centroid blocks P0..P1-1.
template <int DT, int P0, int P1>
__device__ __forceinline__ void mfma_part(typename Fmt<DT>::Acc (&acc)[4][4], const u32x4 (&a)[4],
                                          const u32x4 (&b)[4]) {
  if constexpr (DT == 0) {
#pragma unroll
    for (int q = P0; q < P1; ++q)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
              __uint_as_float(a[mb][q]), __uint_as_float(b[nb][q]), acc[mb][nb], 0, 0, 0);
  } else {
#pragma unroll
    for (int mb = P0; mb < P1; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        if constexpr (kIntSearch<DT>)
          acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a[mb]),
                                                              __builtin_bit_cast(i32x4, b[nb]),
                                                              acc[mb][nb], 0, 0, 0);
        else if constexpr (DT == 1)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, a[mb]), __builtin_bit_cast(bf16x8, b[nb]), acc[mb][nb], 0,
              0, 0);
        else
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[mb]),
                                                               __builtin_bit_cast(f16x8, b[nb]),
                                                               acc[mb][nb], 0, 0, 0);
      }
  }
}

// Bias tile of a panel: lane-group g holds centroids 4 g .. 4 g + 3 of each
// 16-row block. fp32 / bf16: -|c|^2/2, -inf past k (the accumulator's initial
// value). int8: -|q|^2 (added at the fold; centroids past k are skipped).
template <int DT>
__device__ __forceinline__ void panel_bias(const float* bias, int k, int j0, int lane,
                                           typename Fmt<DT>::Acc (&bt)[4]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + mb * 16 + 4 * (lane >> 4) + v;
      if constexpr (kIntSearch<DT>)
        bt[mb][v] = j < k ? reinterpret_cast<const int32_t*>(bias)[j] : 0;
      else
        bt[mb][v] = j < k ? bias[j] : -__builtin_inff();
    }
}

// Folds a finished panel into the running best of each point column. A lane
// holds 16 scores per point column, in increasing centroid order (slot
// (mb, v) is centroid j0 + 16 mb + 4 (lane / 16) + v). It first takes their
// maximum m; only where m beats the running best does it look for the first
// slot holding m, the lowest such index, which is what an ordered walk that
// keeps the first strict maximum finds. Past k the int8 scores are masked
// (float scores are -inf there through the bias).
template <int DT>
__device__ __forceinline__ void fold_panel(const typename Fmt<DT>::Acc (&acc)[4][4],
                                           const typename Fmt<DT>::Acc (&bt)[4], int j0, int k,
                                           int lane, typename Fmt<DT>::Sc (&best)[4],
                                           int (&bidx)[4]) {
  using Sc = typename Fmt<DT>::Sc;
  const int jl = j0 + 4 * (lane >> 4);
  const bool tail = j0 + 64 > k;  // some slot of this wave is past k
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    Sc sc[16];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if constexpr (kIntSearch<DT>) {
          const int x = 2 * acc[mb][nb][v] + bt[mb][v];
          sc[4 * mb + v] = (tail && jl + 16 * mb + v >= k) ? INT32_MIN : x;
        } else {
          sc[4 * mb + v] = acc[mb][nb][v];
        }
      }
    // the largest of the 16: integers by compare and select, floats in a
    // tree of max3 (eight instructions instead of thirty; the scores are
    // finite or -inf, and equal values give the same index below)
    Sc m;
    if constexpr (kIntSearch<DT>) {
      m = sc[0];
#pragma unroll
      for (int q = 1; q < 16; ++q) m = sc[q] > m ? sc[q] : m;
    } else {
      Sc t[8];
#pragma unroll
      for (int q = 0; q < 5; ++q) t[q] = __builtin_fmaxf(__builtin_fmaxf(sc[3 * q], sc[3 * q + 1]), sc[3 * q + 2]);
      t[5] = __builtin_fmaxf(__builtin_fmaxf(t[0], t[1]), t[2]);
      t[6] = __builtin_fmaxf(__builtin_fmaxf(t[3], t[4]), sc[15]);
      m = __builtin_fmaxf(t[5], t[6]);
    }
    if (m > best[nb]) {
      int jb = -1;
#pragma unroll
      for (int q = 15; q >= 0; --q)
        if (sc[q] == m) jb = jl + 16 * (q >> 2) + (q & 3);
      best[nb] = m;
      bidx[nb] = jb;
    }
  }
}

template <int DT>
__device__ __forceinline__ void init_tile(typename Fmt<DT>::Acc (&acc)[4][4],
                                          const typename Fmt<DT>::Acc (&bt)[4]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      if constexpr (kIntSearch<DT>)
        acc[mb][nb] = i32x4{0, 0, 0, 0};
      else
        acc[mb][nb] = bt[mb];
    }
}

// Cross-wave merge and the per-point outputs, shared by both kernels: the
// four lane groups of a point, then the kWM centroid waves through LDS.
// xn = |x|^2; dist = |x|^2 - score (int8: the exact integer |x - q|^2), or
// for fp32 / bf16 |x|^2 - 2 score, clamped at 0; with sim the score is the
// similarity, reported as is, and the error adds 2 - 2 x similarity.
template <int DT>
__device__ __forceinline__ double finish_points(typename Fmt<DT>::Sc (&best)[4], int (&bidx)[4],
                                                typename Fmt<DT>::Sc (*m_s)[kTP],
                                                int (*m_j)[kTP],
                                                const typename Fmt<DT>::Sc* xn_s, int tile0,
                                                int nrows, int k, int32_t* labels, float* dists,
                                                int32_t* counts, int sim) {
  using Sc = typename Fmt<DT>::Sc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    Sc sc = best[nb];
    int j = bidx[nb];
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const Sc os = __shfl_xor(sc, off, 64);
      const int oj = __shfl_xor(j, off, 64);
      if (os > sc || (os == sc && (unsigned)oj < (unsigned)j)) {
        sc = os;
        j = oj;
      }
    }
    if ((lane >> 4) == 0) {
      m_s[wm][wn * 64 + nb * 16 + lane] = sc;
      m_j[wm][wn * 64 + nb * 16 + lane] = j;
    }
  }
  __syncthreads();

  double dsum = 0.0;
  if (tid < kTP) {
    const int p = tid;
    Sc sc = m_s[0][p];
    int j = m_j[0][p];
#pragma unroll
    for (int w = 1; w < kWM; ++w) {
      const Sc s1 = m_s[w][p];
      const int j1 = m_j[w][p];
      if (s1 > sc || (s1 == sc && (unsigned)j1 < (unsigned)j)) {
        sc = s1;
        j = j1;
      }
    }
    if (j < 0 || j >= k) j = 0;  // only reachable with non-finite data
    const int slot = tile0 + p;
    if (slot < nrows) {
      labels[slot] = j;
      if (counts) atomicAdd(&counts[j], 1);
      if constexpr (kIntSearch<DT>) {
        const long long dist = (long long)xn_s[p] - (long long)sc;
        if (dists) dists[slot] = (float)dist;
        dsum = (double)dist;
      } else {
        const float dist = fmaxf(xn_s[p] - 2.0f * sc, 0.0f);
        if (dists) dists[slot] = sim ? sc : dist;
        dsum = sim ? 2.0 - 2.0 * (double)sc : (double)dist;
      }
    }
  }
  return dsum;
}

template <int DT>
__global__ __launch_bounds__(kThreads, 1) void assign_kernel(
    const unsigned char* __restrict__ X, int d, const uint32_t* __restrict__ rows, int nrows,
    const unsigned char* __restrict__ Cs, const float* __restrict__ bias, int k,
    int32_t* __restrict__ labels, float* __restrict__ dists, int32_t* __restrict__ counts,
    double* __restrict__ obj, int sim) {
  using Acc = typename Fmt<DT>::Acc;
  using Sc = typename Fmt<DT>::Sc;
  constexpr int ES = Fmt<DT>::ES;
  constexpr int EPV = 16 / ES;          // elements per 16-byte chunk
  constexpr int EPS = kSlab / ES;       // elements per stage
  __shared__ __attribute__((aligned(16))) unsigned char lx[2][kTP * kStride];
  __shared__ __attribute__((aligned(16))) unsigned char lc[2][kTC * kStride];
  __shared__ Sc m_s[kWM][kTP];
  __shared__ int m_j[kWM][kTP];
  __shared__ Sc xn_s[kTP];
  __shared__ double red[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;  // which 64 centroids of the panel
  const int wn = wave & 1;   // which 64 points of the tile
  const int tile0 = blockIdx.x * kTP;

  // Global->LDS mapping: kChunks threads per row slab. Rows past the end read
  // a valid row (their results are discarded or masked by the bias).
  const int ch = tid % kChunks;
  const int rb = tid / kChunks;
  const size_t rowbytes = (size_t)d * ES;
  const unsigned char* xrow[kXL];
#pragma unroll
  for (int i = 0; i < kXL; ++i) {
    const int slot = min(tile0 + rb + kRowsPerPass * i, nrows - 1);
    const size_t r = rows ? (size_t)rows[slot] : (size_t)slot;
    xrow[i] = X + r * rowbytes;
  }

  const int nst = (d + EPS - 1) / EPS;
  const int npan = (k + kTC - 1) / kTC;

  u32x4 rx[kXL], rc[kCL];
  bool colin = true;  // this thread's chunk of the staged slab lies inside the row
  auto gload = [&](int panel, int s) {
    const int col = s * EPS + ch * EPV;
    colin = col < d;
#pragma unroll
    for (int i = 0; i < kXL; ++i) rx[i] = point_chunk<DT>(load_slab16<DT, false>(xrow[i], col, d));
#pragma unroll
    for (int i = 0; i < kCL; ++i) {
      const int j = min(panel * kTC + rb + kRowsPerPass * i, k - 1);
      rc[i] = load_slab16<DT == 5 ? 2 : DT, false>(Cs + (size_t)j * rowbytes, col, d);
    }
  };
  auto sstore = [&](int buf) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kXL; ++i)
      *reinterpret_cast<u32x4*>(&lx[buf][(rb + kRowsPerPass * i) * kStride + ch * 16]) =
          colin ? rx[i] : z;
#pragma unroll
    for (int i = 0; i < kCL; ++i)
      *reinterpret_cast<u32x4*>(&lc[buf][(rb + kRowsPerPass * i) * kStride + ch * 16]) =
          colin ? rc[i] : z;
  };

  Acc acc[4][4];
  Acc bt[4];
  Sc best[4];
  int bidx[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    best[nb] = kIntSearch<DT> ? (Sc)INT32_MIN : (Sc)-__builtin_inff();
    bidx[nb] = -1;
  }
  Sc xpart[kXL];  // |x|^2 partials of this thread's point-row slabs
#pragma unroll
  for (int i = 0; i < kXL; ++i) xpart[i] = 0;

  // Two LDS stages: the global loads of the next stage are in flight while
  // the MFMAs consume the current one.
  gload(0, 0);
#pragma unroll
  for (int i = 0; i < kXL; ++i) xpart[i] += colin ? sumsq16<DT>(rx[i]) : (Sc)0;
  sstore(0);
  __syncthreads();
  panel_bias<DT>(bias, k, wm * 64, lane, bt);
  init_tile<DT>(acc, bt);

  int panel = 0, s = 0, buf = 0;
  while (true) {
    int np = panel, ns = s + 1;
    if (ns == nst) {
      ns = 0;
      ++np;
    }
    const bool more = np < npan;
    if (more) gload(np, ns);

#pragma unroll
    for (int kk = 0; kk < kSlab / 64; ++kk) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        a[mb] = *reinterpret_cast<const u32x4*>(
            &lc[buf][(wm * 64 + mb * 16 + (lane & 15)) * kStride + kk * 64 + (lane >> 4) * 16]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        b[nb] = *reinterpret_cast<const u32x4*>(
            &lx[buf][(wn * 64 + nb * 16 + (lane & 15)) * kStride + kk * 64 + (lane >> 4) * 16]);
      mfma_slice<DT>(acc, a, b);
    }

    if (ns == 0) {
      // panel complete: fold it into the running best
      fold_panel<DT>(acc, bt, panel * kTC + wm * 64, k, lane, best, bidx);
      if (more) {
        panel_bias<DT>(bias, k, np * kTC + wm * 64, lane, bt);
        init_tile<DT>(acc, bt);
      }
    }
    if (!more) break;
    if (np == 0) {
#pragma unroll
      for (int i = 0; i < kXL; ++i) xpart[i] += colin ? sumsq16<DT>(rx[i]) : (Sc)0;
    }
    sstore(buf ^ 1);
    __syncthreads();
    panel = np;
    s = ns;
    buf ^= 1;
  }

  // |x|^2: fold the column-chunk threads of each point row (adjacent lanes)
#pragma unroll
  for (int i = 0; i < kXL; ++i) {
    Sc v = xpart[i];
#pragma unroll
    for (int o = 1; o < kChunks; o <<= 1) v += __shfl_xor(v, o, 64);
    if (ch == 0) xn_s[rb + kRowsPerPass * i] = v;
  }
  double dsum = finish_points<DT>(best, bidx, m_s, m_j, xn_s, tile0, nrows, k, labels, dists,
                                  counts, sim);
  if (obj) {
    dsum = wave_sum(dsum);
    if (lane == 0) red[wave] = dsum;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
      for (int w = 0; w < kThreads / 64; ++w) t += red[w];
      atomicAdd(obj, t);
    }
  }
}

// ---------------------------------------------------------------------------
// The same tiling for rows made of whole 16-byte chunks, with the stage data
// moved by the direct global-to-LDS path of gfx950 (global_load_lds_dwordx4):
// no register round trip and no LDS store instructions. Three stage buffers
// form a ring, so the loads of stage t + 2 are in flight while the MFMAs
// consume stage t, and one wait plus one barrier close each stage.
//
// A direct load writes the 64 lanes' 16-byte pieces to 1 KB of consecutive
// LDS, i.e. 8 unpadded 128-byte rows per wave load. To keep the MFMA operand
// reads (16 rows, one chunk each) free of bank conflicts the chunk positions
// are swizzled: chunk c of row r sits at position c ^ (r % 8); each lane
// fetches the chunk that belongs at its position. In the last stage of a
// ragged row the chunks past the row end are zeroed in LDS before use, and
// the loads for them read the row's first chunk (in bounds, finite).
// ---------------------------------------------------------------------------
constexpr int kRing = 3;                         // stage buffers
constexpr int kRowsStage = kTP + kTC;            // point rows, then centroid rows
constexpr int kStageBytes = kRowsStage * kSlab;  // 48 KB
constexpr int kLoadsPerWave = kRowsStage / 8 / (kThreads / 64);  // 8-row wave loads

// Chunk position of chunk c in row r. Rows r and r + 8 use different
// positions, so 8 or 16 consecutive rows read at one chunk index touch
// distinct banks whether the LDS serves 8 lanes (32 banks) or 16 lanes (64
// banks) of a 16-byte read per cycle.
__device__ __forceinline__ int swz_pos(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * kSlab + (swz_pos(r, c) << 4); }

template <int DT>
__global__ __launch_bounds__(kThreads, 1) void assign_ring_kernel(
    const unsigned char* __restrict__ X, int d, const uint32_t* __restrict__ rows, int nrows,
    const unsigned char* __restrict__ Cs, const float* __restrict__ bias, int k,
    int32_t* __restrict__ labels, float* __restrict__ dists, int32_t* __restrict__ counts,
    double* __restrict__ obj, int sim) {
  using Acc = typename Fmt<DT>::Acc;
  using Sc = typename Fmt<DT>::Sc;
  constexpr int ES = Fmt<DT>::ES;
  constexpr int EPV = 16 / ES;
  constexpr int EPS = kSlab / ES;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kRing * kStageBytes];
  __shared__ Sc m_s[kWM][kTP];
  __shared__ int m_j[kWM][kTP];
  __shared__ Sc xn_s[kTP];
  __shared__ double red[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int tile0 = blockIdx.x * kTP;
  const size_t rowbytes = (size_t)d * ES;
  const int nst = (d + EPS - 1) / EPS;
  const int npan = (k + kTC - 1) / kTC;
  const int total = nst * npan;

  // Wave loads of this wave: load i covers stage rows 8 g .. 8 g + 7 with
  // g = wave * kLoadsPerWave + i; this lane fills LDS position lane % 8 of
  // row 8 g + lane / 8, i.e. logical chunk swz_pos(row, lane % 8). Stages are
  // issued in order; (ip, is) is the next stage to issue, islot its buffer.
  // Source = row pointer (points: fixed; centroids: per panel) + the stage's
  // column + the lane's chunk.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lr = lane >> 3;
  const bool ragged = d % EPS != 0;
  const unsigned char* rowp[kLoadsPerWave];
  int pcol[kLoadsPerWave];
  auto centroid_row = [&](int panel, int g) {
    const int j = min(panel * kTC + 8 * g - kTP + lr, k - 1);
    return Cs + (size_t)j * rowbytes;
  };
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int g = wv * kLoadsPerWave + i;
    pcol[i] = swz_pos(8 * g + lr, lane & 7) * EPV;
    if (8 * g < kTP) {
      const int slot = min(tile0 + 8 * g + lr, nrows - 1);
      const size_t ri = rows ? (size_t)rows[slot] : (size_t)slot;
      rowp[i] = X + ri * rowbytes;
    } else {
      rowp[i] = centroid_row(0, g);
    }
  }
  int ip = 0, is = 0, islot = 0, issued = 0;
  auto issue_next = [&]() {
    unsigned char* dst = ring + islot * kStageBytes;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int col = is * EPS + pcol[i];
      const int c = ragged && col >= d ? 0 : col;
      lds_load16(rowp[i] + (size_t)c * ES, dst + 1024 * (wv * kLoadsPerWave + i));
    }
    islot = islot + 1 == kRing ? 0 : islot + 1;
    if (issued + 1 < total) {  // past the end the last stage is loaded again
      ++issued;
      if (++is == nst) {
        is = 0;
        ++ip;
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) {
          const int g = wv * kLoadsPerWave + i;
          if (8 * g >= kTP) rowp[i] = centroid_row(ip, g);
        }
      }
    }
  };

  Acc acc[4][4];
  Acc bcur[4], bnext[4];  // bias tiles of the current and the next panel
  auto load_bias = [&](int panel) { panel_bias<DT>(bias, k, panel * kTC + wm * 64, lane, bnext); };

  Sc best[4];
  int bidx[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    best[nb] = kIntSearch<DT> ? (Sc)INT32_MIN : (Sc)-__builtin_inff();
    bidx[nb] = -1;
  }
  // |x|^2 partials: thread (rb, ch) covers chunk ch of point rows rb + kRowsPerPass i
  const int ch = tid & 7, rb = tid >> 3;
  constexpr int kXR = kTP / kRowsPerPass;
  Sc xpart[kXR];
#pragma unroll
  for (int i = 0; i < kXR; ++i) xpart[i] = 0;

  load_bias(0);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) bcur[mb] = bnext[mb];
  init_tile<DT>(acc, bcur);
  // Exactly kLoadsPerWave ring loads are issued per stage (the last stages
  // reload the final stage into a buffer that is no longer read), so "the
  // previous stage's loads are done" is always vmcnt <= kLoadsPerWave.
  issue_next();
  issue_next();
  EMK_WAIT_VMCNT(kLoadsPerWave);
  lds_barrier();

  if constexpr (DT == 3) {
    int panel = 0, s = 0, cslot = 0;
    for (int t = 0; t < total; ++t) {
      const bool last_s = s == nst - 1;
      const bool more_p = panel + 1 < npan;
      if (last_s && more_p) load_bias(panel + 1);  // before the ring loads: retired by the stage wait
      unsigned char* cur = ring + cslot * kStageBytes;
      if (ragged && last_s) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int q = tid; q < kRowsStage * kChunks; q += kThreads) {
          const int r = q >> 3, c = q & 7;
          if (s * EPS + c * EPV >= d) *reinterpret_cast<u32x4*>(cur + swz(r, c)) = z;
        }
        lds_barrier();
      }
      if (panel == 0) {
        const bool in = s * EPS + ch * EPV < d;
#pragma unroll
        for (int i = 0; i < kXR; ++i)
          if (in)
            xpart[i] += sumsq16<DT>(point_chunk<DT>(
                *reinterpret_cast<const u32x4*>(cur + swz(rb + kRowsPerPass * i, ch))));
      }
      static_assert(kSlab == 128, "one 16x16x128 FP8 MFMA per stage");
      u32x4 a[2][4], b[2][4];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int pc = swz_pos(lane & 15, kk * 4 + (lane >> 4)) << 4;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          a[kk][mb] = *reinterpret_cast<const u32x4*>(
              cur + (kTP + wm * 64 + mb * 16 + (lane & 15)) * kSlab + pc);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          b[kk][nb] = *reinterpret_cast<const u32x4*>(
              cur + (wn * 64 + nb * 16 + (lane & 15)) * kSlab + pc);
      }
      mfma_stage_f8(acc, a, b);
      // the loads of stage t + 2, issued while the matrix core works on this stage
      issue_next();
      if (last_s) {
        fold_panel<DT>(acc, bcur, panel * kTC + wm * 64, k, lane, best, bidx);
        if (more_p) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) bcur[mb] = bnext[mb];
          init_tile<DT>(acc, bcur);
        }
      }
      // the next stage's loads have landed in LDS for this wave, then for all
      EMK_WAIT_VMCNT(kLoadsPerWave);
      lds_barrier();
      cslot = cslot + 1 == kRing ? 0 : cslot + 1;
      if (last_s) {
        s = 0;
        ++panel;
      } else {
        ++s;
      }
    }
  } else {
    // Each stage: the MFMAs of its first 64-byte slice, the loads of stage
    // t + 2, then part of the second slice's MFMAs before the stage's wait and
    // barrier and the rest after it, while the fragments of the next stage's
    // first slice are read (they cover that read's latency, which otherwise
    // idles every wave at once after each barrier). The panel's fold follows
    // its last MFMAs.
    const int pc0 = swz_pos(lane & 15, lane >> 4) << 4;  // rows are 16-aligned + lane % 16
    const int pc1 = swz_pos(lane & 15, 4 + (lane >> 4)) << 4;
    auto read_frags = [&](const unsigned char* base, int pc, u32x4 (&a)[4], u32x4 (&b)[4]) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        a[mb] = *reinterpret_cast<const u32x4*>(base + (kTP + wm * 64 + mb * 16 + (lane & 15)) * kSlab + pc);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        b[nb] = point_chunk<DT>(
            *reinterpret_cast<const u32x4*>(base + (wn * 64 + nb * 16 + (lane & 15)) * kSlab + pc));
    };
    static_assert(kSlab == 128, "two 64-byte slices per stage");
    // MFMAs of the second slice run before the barrier: fp32 k-steps 0..2 of
    // 4 (48 of 64); the others none of their 16
    constexpr int kSplit = DT == 0 ? 3 : 0;
    u32x4 fa0[4], fb0[4], fa1[4], fb1[4];
    read_frags(ring, pc0, fa0, fb0);
    int panel = 0, s = 0, cslot = 0;
    for (int t = 0; t < total; ++t) {
      const bool last_s = s == nst - 1;
      const bool more_p = panel + 1 < npan;
      if (last_s && more_p) load_bias(panel + 1);  // before the ring loads: retired by the stage wait
      unsigned char* cur = ring + cslot * kStageBytes;
      if (ragged && last_s) {
        // zero the chunks past the row end (points and centroids), then read
        // the first slice again
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int q = tid; q < kRowsStage * kChunks; q += kThreads) {
          const int r = q >> 3, c = q & 7;
          if (s * EPS + c * EPV >= d) *reinterpret_cast<u32x4*>(cur + swz(r, c)) = z;
        }
        lds_barrier();
        read_frags(cur, pc0, fa0, fb0);
      }
      if (panel == 0) {
        const bool in = s * EPS + ch * EPV < d;
#pragma unroll
        for (int i = 0; i < kXR; ++i)
          if (in)
            xpart[i] += sumsq16<DT>(point_chunk<DT>(
                *reinterpret_cast<const u32x4*>(cur + swz(rb + kRowsPerPass * i, ch))));
      }
      read_frags(cur, pc1, fa1, fb1);
      mfma_slice<DT>(acc, fa0, fb0);
      // the loads of stage t + 2, into the buffer of stage t - 1 (its reads
      // all ended before the barrier that opened this stage)
      issue_next();
      mfma_part<DT, 0, kSplit>(acc, fa1, fb1);
      // the next stage's loads have landed in LDS for this wave, then for all
      __builtin_amdgcn_sched_barrier(0);
      EMK_WAIT_VMCNT(kLoadsPerWave);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      cslot = cslot + 1 == kRing ? 0 : cslot + 1;
      if (t + 1 < total) read_frags(ring + cslot * kStageBytes, pc0, fa0, fb0);
      mfma_part<DT, kSplit, 4>(acc, fa1, fb1);
      if (last_s) {
        // panel complete: fold it into the running best (centroids in increasing order)
        fold_panel<DT>(acc, bcur, panel * kTC + wm * 64, k, lane, best, bidx);
        if (more_p) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) bcur[mb] = bnext[mb];
          init_tile<DT>(acc, bcur);
        }
        s = 0;
        ++panel;
      } else {
        ++s;
      }
    }
  }

  EMK_WAIT_VMCNT(0);  // no ring load may still be writing LDS at exit

  // |x|^2: fold the eight chunk threads of each point row (adjacent lanes)
#pragma unroll
  for (int i = 0; i < kXR; ++i) {
    Sc v = xpart[i];
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) v += __shfl_xor(v, o, 64);
    if (ch == 0) xn_s[rb + kRowsPerPass * i] = v;
  }
  double dsum = finish_points<DT>(best, bidx, m_s, m_j, xn_s, tile0, nrows, k, labels, dists,
                                  counts, sim);
  if (obj) {
    dsum = wave_sum(dsum);
    if (lane == 0) red[wave] = dsum;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
      for (int w = 0; w < kThreads / 64; ++w) t += red[w];
      atomicAdd(obj, t);
    }
  }
}

}  // namespace

hipError_t launch_assign(int dt, const void* X, int d, const uint32_t* rows, int nrows,
                         const void* Cs, const float* bias, int k, int32_t* labels, float* dists,
                         int32_t* counts, double* obj, bool sim, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  if ((dt == 1 || dt == 4) && assign_bf16_resident_ok(d, X, Cs))
    return launch_assign_bf16_resident(X, d, rows, nrows, Cs, bias, k, labels, dists, counts, obj,
                                       sim, dt == 4, st);
  if (dt == 3 && !sim && assign_f8_wide_ok(d, X, Cs))
    return launch_assign_f8_wide(X, d, rows, nrows, Cs, bias, k, labels, dists, counts, obj, st);
  if ((dt == 2 || dt == 5) && !sim && assign_i8_wide_ok(d, X, Cs))
    return launch_assign_i8_wide(X, d, rows, nrows, Cs, bias, k, labels, dists, counts, obj,
                                 dt == 5, st);
  if ((dt == 2 || dt == 5) && !sim && assign_i8_resident_ok(d, X, Cs))
    return launch_assign_i8_resident(X, d, rows, nrows, Cs, bias, k, labels, dists, counts, obj,
                                     dt == 5, st);
  const dim3 grid((nrows + kTP - 1) / kTP), block(kThreads);
  const auto* x = static_cast<const unsigned char*>(X);
  const auto* c = static_cast<const unsigned char*>(Cs);
  const bool aligned = ((uintptr_t)X % 16 == 0) && ((uintptr_t)Cs % 16 == 0);
  const int epv = (dt == 2 || dt == 3 || dt == 5) ? 16 : (dt == 1 || dt == 4) ? 8 : 4;
  const bool ring = aligned && d % epv == 0;
  const int sm = sim ? 1 : 0;
#define EMK_ASSIGN(KERNEL) \
  KERNEL<<<grid, block, 0, st>>>(x, d, rows, nrows, c, bias, k, labels, dists, counts, obj, sm)
  if (dt == 5) {
    if (ring)
      EMK_ASSIGN(assign_ring_kernel<5>);
    else
      EMK_ASSIGN(assign_kernel<5>);
  } else if (dt == 4) {
    if (ring)
      EMK_ASSIGN(assign_ring_kernel<4>);
    else
      EMK_ASSIGN(assign_kernel<4>);
  } else if (dt == 3) {
    if (ring)
      EMK_ASSIGN(assign_ring_kernel<3>);
    else
      EMK_ASSIGN(assign_kernel<3>);
  } else if (dt == 2) {
    if (ring)
      EMK_ASSIGN(assign_ring_kernel<2>);
    else
      EMK_ASSIGN(assign_kernel<2>);
  } else if (dt == 1) {
    if (ring)
      EMK_ASSIGN(assign_ring_kernel<1>);
    else
      EMK_ASSIGN(assign_kernel<1>);
  } else {
    if (ring)
      EMK_ASSIGN(assign_ring_kernel<0>);
    else
      EMK_ASSIGN(assign_kernel<0>);
  }
#undef EMK_ASSIGN
  return hipGetLastError();
}

}  // namespace emk
