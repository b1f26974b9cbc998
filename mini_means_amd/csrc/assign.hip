// Fused nearest-centroid assignment for gfx950 (MFMA, wave64).
//
// A workgroup owns a tile of TP points and sweeps every centroid in panels of
// TC. For each (panel, d-chunk) the point rows and centroid rows are staged
// through LDS (double buffered, one 128-byte slab per row); four waves each
// compute a 64 x 64 block of scores with 16x16 MFMA tiles:
//   fp32 X: v_mfma_f32_16x16x4_f32     bf16 X: v_mfma_f32_16x16x32_bf16.
// Centroids sit on the MFMA M dimension and points on N, so after a tile each
// lane holds four centroid scores of a single point; the running best score
// and its index stay in registers across all panels and are merged across the
// four lane groups with cross-lane shuffles and across the two M-waves through
// LDS only once at the end. The score is x.c - |c|^2/2: the bias -|c|^2/2 is
// the accumulator's initial value, so the argmax needs compares only, and the
// squared distance is |x|^2 - 2 * best. No n x k distance matrix is formed.
//
// Ties: each lane visits its centroids in increasing index order and keeps
// the first strict maximum; merges prefer the lower index on equal scores, so
// the lowest index wins overall, matching argmin over the squared distance.
#include "kernels.hpp"

namespace emk {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kTP = 128;       // points per workgroup
constexpr int kTC = 128;       // centroids per panel
constexpr int kSlab = 128;     // bytes of one row per stage
constexpr int kStride = 144;   // LDS row pitch in bytes (slab + 16 to spread banks)
constexpr int kThreads = 256;

template <bool BF16, bool VEC>
__device__ __forceinline__ u32x4 load_slab16(const unsigned char* row, int col, int d) {
  // 16 bytes of a row starting at element `col`; zero past the end of the row.
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row == nullptr) return v;
  if constexpr (VEC) {
    if (col < d) v = *reinterpret_cast<const u32x4*>(row + (size_t)col * ES);
  } else {
    if constexpr (BF16) {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(row);
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int c = col + e;
        const uint32_t h = c < d ? (uint32_t)p[c] : 0u;
        w[e >> 1] |= h << (16 * (e & 1));
      }
      v = u32x4{w[0], w[1], w[2], w[3]};
    } else {
      const float* p = reinterpret_cast<const float*>(row);
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = (col + e) < d ? p[col + e] : 0.0f;
      v = u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                __float_as_uint(f[3])};
    }
  }
  return v;
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void assign_kernel(
    const unsigned char* __restrict__ X, int d, const uint32_t* __restrict__ rows, int nrows,
    const unsigned char* __restrict__ Cs, const float* __restrict__ bias, int k,
    int32_t* __restrict__ labels, float* __restrict__ dists, int32_t* __restrict__ counts,
    double* __restrict__ obj) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;          // elements per 16-byte chunk
  constexpr int EPS = kSlab / ES;       // elements per stage
  __shared__ __attribute__((aligned(16))) unsigned char lx[2][kTP * kStride];
  __shared__ __attribute__((aligned(16))) unsigned char lc[2][kTC * kStride];
  __shared__ float m_s[2][kTP];
  __shared__ int m_j[2][kTP];
  __shared__ float xn_s[kTP];
  __shared__ double red[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;  // which 64 centroids of the panel
  const int wn = wave & 1;   // which 64 points of the tile
  const int tile0 = blockIdx.x * kTP;

  // Global->LDS mapping: 8 threads per 128-byte row slab, 32 rows per pass.
  const int ch = tid & 7;
  const int rb = tid >> 3;
  const size_t rowbytes = (size_t)d * ES;
  const unsigned char* xrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = tile0 + rb + 32 * i;
    if (slot < nrows) {
      const size_t r = rows ? (size_t)rows[slot] : (size_t)slot;
      xrow[i] = X + r * rowbytes;
    } else {
      xrow[i] = nullptr;
    }
  }

  const int nst = (d + EPS - 1) / EPS;
  const int npan = (k + kTC - 1) / kTC;
  const int total = nst * npan;

  u32x4 rx[4], rc[4];
  auto gload = [&](int it) {
    const int panel = it / nst;
    const int s = it - panel * nst;
    const int col = s * EPS + ch * EPV;
#pragma unroll
    for (int i = 0; i < 4; ++i) rx[i] = load_slab16<BF16, VEC>(xrow[i], col, d);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = panel * kTC + rb + 32 * i;
      rc[i] = load_slab16<BF16, VEC>(j < k ? Cs + (size_t)j * rowbytes : nullptr, col, d);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&lx[buf][(rb + 32 * i) * kStride + ch * 16]) = rx[i];
      *reinterpret_cast<u32x4*>(&lc[buf][(rb + 32 * i) * kStride + ch * 16]) = rc[i];
    }
  };

  f32x4 acc[4][4];
  auto init_acc = [&](int panel) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      f32x4 b;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = panel * kTC + wm * 64 + mb * 16 + 4 * (lane >> 4) + v;
        b[v] = j < k ? bias[j] : -__builtin_inff();
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = b;
    }
  };

  float best[4];
  int bidx[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    best[nb] = -__builtin_inff();
    bidx[nb] = -1;
  }
  float xpart = 0.0f;  // |x|^2 partial: point tid/2, half tid&1 of each slab

  gload(0);
  sstore(0);
  __syncthreads();
  init_acc(0);

  for (int it = 0; it < total; ++it) {
    const int panel = it / nst;
    const int s = it - panel * nst;
    const int buf = it & 1;
    if (it + 1 < total) gload(it + 1);

#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        a[mb] = *reinterpret_cast<const u32x4*>(
            &lc[buf][(wm * 64 + mb * 16 + (lane & 15)) * kStride + kk * 64 + (lane >> 4) * 16]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        b[nb] = *reinterpret_cast<const u32x4*>(
            &lx[buf][(wn * 64 + nb * 16 + (lane & 15)) * kStride + kk * 64 + (lane >> 4) * 16]);
      if constexpr (BF16) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a[mb]), __builtin_bit_cast(bf16x8, b[nb]),
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

    if (panel == 0) {
      const unsigned char* p = &lx[buf][(tid >> 1) * kStride + (tid & 1) * 64];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p + 16 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (BF16) {
            const float lo = __uint_as_float(w[e] << 16);
            const float hi = __uint_as_float(w[e] & 0xFFFF0000u);
            xpart += lo * lo + hi * hi;
          } else {
            const float f = __uint_as_float(w[e]);
            xpart += f * f;
          }
        }
      }
    }

    if (s == nst - 1) {
      // fold this panel into the running best (centroids in increasing order)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float sc = acc[mb][nb][v];
            if (sc > best[nb]) {
              best[nb] = sc;
              bidx[nb] = panel * kTC + wm * 64 + mb * 16 + 4 * (lane >> 4) + v;
            }
          }
      if (panel + 1 < npan) init_acc(panel + 1);
    }

    if (it + 1 < total) sstore(buf ^ 1);
    __syncthreads();
  }

  // merge the four lane groups that share a point
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    float sc = best[nb];
    int j = bidx[nb];
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float os = __shfl_xor(sc, off, 64);
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
  xpart += __shfl_xor(xpart, 1, 64);
  if ((tid & 1) == 0) xn_s[tid >> 1] = xpart;
  __syncthreads();

  double dsum = 0.0;
  if (tid < kTP) {
    const int p = tid;
    float sc = m_s[0][p];
    int j = m_j[0][p];
    const float s1 = m_s[1][p];
    const int j1 = m_j[1][p];
    if (s1 > sc || (s1 == sc && (unsigned)j1 < (unsigned)j)) {
      sc = s1;
      j = j1;
    }
    if (j < 0 || j >= k) j = 0;  // only reachable with non-finite data
    const int slot = tile0 + p;
    if (slot < nrows) {
      const float dist = fmaxf(xn_s[p] - 2.0f * sc, 0.0f);
      labels[slot] = j;
      if (dists) dists[slot] = dist;
      if (counts) atomicAdd(&counts[j], 1);
      dsum = (double)dist;
    }
  }
  if (obj) {
    dsum = wave_sum(dsum);
    if (lane == 0) red[wave] = dsum;
    __syncthreads();
    if (tid == 0) atomicAdd(obj, red[0] + red[1] + red[2] + red[3]);
  }
}

}  // namespace

hipError_t launch_assign(bool bf16, const void* X, int d, const uint32_t* rows, int nrows,
                         const void* Cs, const float* bias, int k, int32_t* labels, float* dists,
                         int32_t* counts, double* obj, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  const dim3 grid((nrows + kTP - 1) / kTP), block(kThreads);
  const auto* x = static_cast<const unsigned char*>(X);
  const auto* c = static_cast<const unsigned char*>(Cs);
  const bool aligned = ((uintptr_t)X % 16 == 0) && ((uintptr_t)Cs % 16 == 0);
  if (bf16) {
    if (aligned && d % 8 == 0)
      assign_kernel<true, true><<<grid, block, 0, st>>>(x, d, rows, nrows, c, bias, k, labels,
                                                        dists, counts, obj);
    else
      assign_kernel<true, false><<<grid, block, 0, st>>>(x, d, rows, nrows, c, bias, k, labels,
                                                         dists, counts, obj);
  } else {
    if (aligned && d % 4 == 0)
      assign_kernel<false, true><<<grid, block, 0, st>>>(x, d, rows, nrows, c, bias, k, labels,
                                                         dists, counts, obj);
    else
      assign_kernel<false, false><<<grid, block, 0, st>>>(x, d, rows, nrows, c, bias, k, labels,
                                                          dists, counts, obj);
  }
  return hipGetLastError();
}

}  // namespace emk
