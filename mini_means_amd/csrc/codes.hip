// INT8 and FP8 (E4M3) codes of fp32 data (README "Data precision"):
// calibration of a per-dimension shift and one power-of-two scale from sample
// rows, encoding of rows into codes, decoding of code-space centroids. All
// three are HBM-bound elementwise or column-reduction kernels.
//
// Calibration: the shift of dimension j is the midrange (min + max) / 2 of
// the sample's column j (fp64, stored as fp32); r is the largest distance of
// a sample value from its shift (fp64); the scale is the largest power of two
// s with s r <= L (L = 127 for int8, 448 for FP8; s = 1 when r = 0).
// Encoding: y = (x - shift) * s with the subtraction and the product in fp32
// (the product by a power of two is exact); int8: clamp(rint(y), -127, 127);
// FP8: the nearest E4M3 value, saturating at +-448; ties to even in both.
// Decoding: c / s + shift in fp64, stored as fp32.
#include "kernels.hpp"

namespace emk {

namespace {

constexpr int kCalCols = 256;     // columns per calibration block
constexpr int kCalRows = 512;     // sample rows per calibration block

// Partial column min / max over rows [blockIdx.x * kCalRows, +kCalRows):
// consecutive threads read consecutive columns of a row (coalesced).
__global__ __launch_bounds__(kCalCols) void minmax_partial_kernel(const float* __restrict__ X,
                                                                  int64_t n, int d,
                                                                  float* __restrict__ pmin,
                                                                  float* __restrict__ pmax) {
  const int col = blockIdx.y * kCalCols + threadIdx.x;
  if (col >= d) return;
  const int64_t r0 = (int64_t)blockIdx.x * kCalRows;
  const int64_t r1 = r0 + kCalRows < n ? r0 + kCalRows : n;
  float mn = __builtin_inff(), mx = -__builtin_inff();
  int64_t r = r0;
  for (; r + 4 <= r1; r += 4) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = X[(r + u) * d + col];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      mn = fminf(mn, v[u]);
      mx = fmaxf(mx, v[u]);
    }
  }
  for (; r < r1; ++r) {
    const float v = X[r * d + col];
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  pmin[(size_t)blockIdx.x * d + col] = mn;
  pmax[(size_t)blockIdx.x * d + col] = mx;
}

// Column min / max over the partials, the shift, and the largest radius of
// the block's columns (fp64) into rpart[blockIdx.x].
__global__ __launch_bounds__(256) void calib_finish_kernel(const float* __restrict__ pmin,
                                                           const float* __restrict__ pmax,
                                                           int nchunks, int d,
                                                           float* __restrict__ shift,
                                                           double* __restrict__ rpart) {
  __shared__ double red[4];
  const int col = blockIdx.x * 256 + threadIdx.x;
  double r = 0.0;
  if (col < d) {
    float mn = __builtin_inff(), mx = -__builtin_inff();
    for (int c = 0; c < nchunks; ++c) {
      mn = fminf(mn, pmin[(size_t)c * d + col]);
      mx = fmaxf(mx, pmax[(size_t)c * d + col]);
    }
    const float s = (float)(((double)mn + (double)mx) / 2.0);
    shift[col] = s;
    const double s64 = (double)s;
    r = fmax((double)mx - s64, s64 - (double)mn);
  }
  r = wave_max(r);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = r;
  __syncthreads();
  if (threadIdx.x == 0) rpart[blockIdx.x] = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
}

// r = the largest of the nparts block radii; the largest power of two s with
// s r <= L. With r = m 2^E and L = mL 2^EL (m, mL in [0.5, 1)), s = 2^e maps
// r to m 2^(E + e), which is <= L for E + e = EL exactly when m <= mL, and
// always for E + e = EL - 1.
__global__ __launch_bounds__(256) void calib_scale_kernel(const double* __restrict__ rpart,
                                                          int nparts, double bound,
                                                          double* scale) {
  __shared__ double red[4];
  double r = 0.0;
  for (int i = threadIdx.x; i < nparts; i += 256) r = fmax(r, rpart[i]);
  r = wave_max(r);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x) return;
  r = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  if (!(r > 0.0)) {
    *scale = 1.0;
    return;
  }
  int E, EL;
  const double m = frexp(r, &E);
  const double mL = frexp(bound, &EL);
  const int e = (m <= mL ? EL : EL - 1) - E;
  *scale = ldexp(1.0, e);
}

// One code (as its byte): FMT 0 int8, 1 FP8 E4M3.
template <int FMT>
__device__ __forceinline__ uint32_t encode_one(float x, float sh, float sc) {
  const float y = __fmul_rn(__fsub_rn(x, sh), sc);
  if constexpr (FMT == 1) return f32_to_e4m3(y);
  return (uint32_t)(uint8_t)(int8_t)fminf(fmaxf(__builtin_rintf(y), -127.0f), 127.0f);
}

// Thread i encodes the 16 consecutive elements [16 i, 16 i + 16) of the flat
// n x d array (VEC: four 16-byte loads, one 16-byte store); the thread past
// the last whole group takes the remaining tail.
template <bool VEC, int FMT>
__global__ __launch_bounds__(256) void encode_kernel(const float* __restrict__ X, int64_t total,
                                                     int d, const float* __restrict__ shift,
                                                     float sc, uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t e0 = i * 16;
  if (e0 >= total) return;
  int col = (int)(e0 % d);
  if (VEC && e0 + 16 <= total) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    f32x4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = reinterpret_cast<const f32x4*>(X + e0)[q];
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        w[q] |= encode_one<FMT>(v[q][u], shift[col], sc) << (8 * u);
        if (++col == d) col = 0;
      }
    *reinterpret_cast<u32x4*>(out + e0) = u32x4{w[0], w[1], w[2], w[3]};
    return;
  }
  const int64_t e1 = e0 + 16 < total ? e0 + 16 : total;
  for (int64_t e = e0; e < e1; ++e) {
    out[e] = (uint8_t)encode_one<FMT>(X[e], shift[col], sc);
    if (++col == d) col = 0;
  }
}

__global__ __launch_bounds__(256) void decode_kernel(const float* __restrict__ C, int64_t total,
                                                     int d, const float* __restrict__ shift,
                                                     double sc, float* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  out[e] = (float)((double)C[e] / sc + (double)shift[e % d]);
}

}  // namespace

size_t calib_workspace_floats(int64_t n, int d) {
  const int64_t chunks = (n + kCalRows - 1) / kCalRows;
  return (size_t)chunks * d * 2 + 2 * (size_t)((d + 255) / 256);  // partials, block radii
}

hipError_t launch_calibrate(const float* X, int64_t n, int d, float* shift, float* work,
                            double bound, double* scale, hipStream_t st) {
  const int chunks = (int)((n + kCalRows - 1) / kCalRows);
  const int nparts = (d + 255) / 256;
  float* pmin = work;
  float* pmax = work + (size_t)chunks * d;
  double* rpart = reinterpret_cast<double*>(pmax + (size_t)chunks * d);
  minmax_partial_kernel<<<dim3(chunks, (d + kCalCols - 1) / kCalCols), kCalCols, 0, st>>>(
      X, n, d, pmin, pmax);
  calib_finish_kernel<<<nparts, 256, 0, st>>>(pmin, pmax, chunks, d, shift, rpart);
  calib_scale_kernel<<<1, 256, 0, st>>>(rpart, nparts, bound, scale);
  return hipGetLastError();
}

hipError_t launch_encode(const float* X, int64_t n, int d, const float* shift, float scale,
                         int fmt, uint8_t* codes, hipStream_t st) {
  const int64_t total = n * (int64_t)d;
  if (total <= 0) return hipSuccess;
  const int64_t threads = (total + 15) / 16;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  const bool vec = (uintptr_t)X % 16 == 0 && (uintptr_t)codes % 16 == 0;
  if (fmt == 1) {
    if (vec)
      encode_kernel<true, 1><<<grid, block, 0, st>>>(X, total, d, shift, scale, codes);
    else
      encode_kernel<false, 1><<<grid, block, 0, st>>>(X, total, d, shift, scale, codes);
  } else {
    if (vec)
      encode_kernel<true, 0><<<grid, block, 0, st>>>(X, total, d, shift, scale, codes);
    else
      encode_kernel<false, 0><<<grid, block, 0, st>>>(X, total, d, shift, scale, codes);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const float* C, int64_t k, int d, const float* shift, double scale,
                         float* out, hipStream_t st) {
  const int64_t total = k * (int64_t)d;
  if (total <= 0) return hipSuccess;
  decode_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(C, total, d, shift, scale, out);
  return hipGetLastError();
}

}  // namespace emk
