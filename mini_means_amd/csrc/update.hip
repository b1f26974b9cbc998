// Everything of an e-means step after the assignment: batch sampling, the
// bucketing of the batch by label, the per-cluster sums, the EMA update of the
// running statistics, dead-cluster revival and the closing mean.
//
// Precision (faiss e_means README, "Data precision"): running counts, running
// sums and centroids are fp32. The running count update is written as
// fl(fl(b*N) + fl(a*n)) with b = fl(1 - a) and no fused multiply-add, so that
// given the same labels it is reproducible bit for bit.
#include "kernels.hpp"

namespace emk {

namespace {

constexpr float kSplitEps = 0x1.0p-10f;  // relative perturbation of a split

constexpr int kNarrowRows = 256;  // rows per grouping work item for rows of at most 1 KB

// Each thread produces q consecutive slots of the batch. A loop trip takes one
// Feistel evaluation of the slot in hand; the thread moves on to its next slot
// as soon as the value lands in [0, n). A wave therefore runs for the largest
// sum of q cycle-walk lengths among its lanes rather than q times the longest
// single walk (walks are geometric, with mean up to 4 when n is just above a
// power of four).
__global__ __launch_bounds__(256) void sample_rows_kernel(PermKey pk, uint64_t start, int count,
                                                          int q, uint32_t* rows) {
  const int64_t base = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * q;
  if (base >= count) return;
  const int qn = (int)(count - base < q ? count - base : q);
  int i = 0;
  uint64_t v = start + (uint64_t)base;
  while (i < qn) {
    v = feistel(v, pk);
    if (v < pk.n) {
      rows[base + i] = (uint32_t)v;
      ++i;
      v = start + (uint64_t)(base + i);
    }
  }
}

__global__ void sample_rows_i32_kernel(PermKey pk, uint64_t start, int count, int32_t* rows) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < count) rows[r] = (int32_t)perm_at(start + (uint64_t)r, pk);
}

// A value in a search format of fp32 data (README "Data precision", convert
// on the fly): y = (x - shift) * scale in fp32, the product by a power of two
// exact, then the nearest bf16 (FMT 1) or fp16 (FMT 4) bits, or the nearest
// E4M3 code (FMT 3, saturating).
template <int FMT>
__device__ __forceinline__ uint32_t to_search_fmt(float y) {
  if constexpr (FMT == 3) return f32_to_e4m3(y);
  else if constexpr (FMT == 4) return f32_to_f16_rne(y);
  else return f32_to_bf16_rne(y);
}

// out[r] = the batch row X[rows[r]] in search format FMT (rows NULL: row r),
// contiguous; shift NULL means 0. Eight elements per thread when rows are
// whole 32-byte chunks, else one.
template <int FMT, bool VEC>
__global__ __launch_bounds__(256) void convert_rows_kernel(const float* __restrict__ X, int d,
                                                           const uint32_t* __restrict__ rows,
                                                           int nrows,
                                                           const float* __restrict__ shift,
                                                           float scale,
                                                           unsigned char* __restrict__ out) {
  constexpr int E = VEC ? 8 : 1;
  constexpr int OB = FMT == 3 ? 1 : 2;  // output bytes per element
  const int per = d / E;
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= (int64_t)nrows * per) return;
  const int r = (int)(q / per), c = (int)(q - (int64_t)r * per) * E;
  const size_t src = (size_t)(rows ? rows[r] : (uint32_t)r) * d + c;
  const size_t dst = ((size_t)r * d + c) * OB;
  if constexpr (VEC) {
    const float4 a = *reinterpret_cast<const float4*>(X + src);
    const float4 b = *reinterpret_cast<const float4*>(X + src + 4);
    float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    if (shift) {
      const float4 sa = *reinterpret_cast<const float4*>(shift + c);
      const float4 sb = *reinterpret_cast<const float4*>(shift + c + 4);
      const float sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = f[e] - sv[e];
    }
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = to_search_fmt<FMT>(f[e] * scale);
    if constexpr (FMT == 3) {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0 |= h[e] << (8 * e);
        w1 |= h[e + 4] << (8 * e);
      }
      *reinterpret_cast<uint2*>(out + dst) = make_uint2(w0, w1);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = h[2 * e] | (h[2 * e + 1] << 16);
      *reinterpret_cast<uint4*>(out + dst) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    const float y = (shift ? X[src] - shift[c] : X[src]) * scale;
    if constexpr (FMT == 3)
      out[dst] = (unsigned char)to_search_fmt<FMT>(y);
    else
      *reinterpret_cast<uint16_t*>(out + dst) = (uint16_t)to_search_fmt<FMT>(y);
  }
}

// The search copy of a centroid coordinate c of fp32 data converted on the
// fly: (c - shift[e]) * scale (shift NULL: c * scale), before rounding.
__device__ __forceinline__ float conv_in(float c, const float* sshift, float sscale, size_t e) {
  return (sshift ? c - sshift[e] : c) * sscale;
}

// Spherical e-means: rescale a row of length d to norm 1 in place, the norm
// and the quotient in fp64 (stored fp32); a zero row stays zero. One wave.
__device__ __forceinline__ void wave_normalize(float* c, int d, int lane) {
  double s2 = 0.0;
  for (int e = lane; e < d; e += 64) {
    const double v = (double)c[e];
    s2 += v * v;
  }
  s2 = wave_sum(s2);
  if (s2 > 0.0) {
    const double nr = sqrt(s2);
    for (int e = lane; e < d; e += 64) c[e] = (float)((double)c[e] / nr);
  }
}

// int8 search code of a code-space centroid value: nearest (ties to even),
// clamped to [-127, 127].
__device__ __forceinline__ int8_t to_code_i8(float c) {
  return (int8_t)fminf(fmaxf(__builtin_rintf(c), -127.0f), 127.0f);
}

// Search code of a centroid of uint8 data: the nearest uint8 value (ties to
// even, clamped to [0, 255]) shifted by -128 into int8, the form the integer
// search compares the shifted rows with.
__device__ __forceinline__ int8_t to_code_u8(float c) {
  return (int8_t)((int)fminf(fmaxf(__builtin_rintf(c), 0.0f), 255.0f) - 128);
}

__device__ __forceinline__ int8_t to_code(float c, bool u8) {
  return u8 ? to_code_u8(c) : to_code_i8(c);
}

// One wave per centroid: C[j] = X[pi(j)] converted to fp32 (rescaled to norm
// 1 for spherical e-means).
__global__ __launch_bounds__(256) void init_centroids_kernel(const unsigned char* X, int dt,
                                                             int d, PermKey pk, int k, float* C,
                                                             int sph) {
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= k) return;
  uint64_t row = 0;
  if (lane == 0) row = perm_at((uint64_t)j, pk);
  row = __shfl(row, 0, 64);
  for (int e = lane; e < d; e += 64) {
    float v;
    if (dt == 1)
      v = bf16_to_f32(reinterpret_cast<const uint16_t*>(X)[row * (uint64_t)d + e]);
    else if (dt == 2)
      v = (float)reinterpret_cast<const int8_t*>(X)[row * (uint64_t)d + e];
    else if (dt == 3)
      v = e4m3_to_f32(reinterpret_cast<const uint8_t*>(X)[row * (uint64_t)d + e]);
    else if (dt == 4)
      v = f16_to_f32(reinterpret_cast<const uint16_t*>(X)[row * (uint64_t)d + e]);
    else if (dt == 5)
      v = (float)X[row * (uint64_t)d + e];
    else
      v = reinterpret_cast<const float*>(X)[row * (uint64_t)d + e];
    C[(size_t)j * d + e] = v;
  }
  if (sph) wave_normalize(C + (size_t)j * d, d, lane);
}

// One wave per centroid: bias = -|c|^2/2 in the search format, Chat = bf16(c)
// (bf16 search) or fp16(c) (fp16 data, hf), Cq = int8 codes of c (int8 data;
// uint8 data, u8: the shifted uint8 codes) or Cf = E4M3 codes of c (FP8 data).
__global__ __launch_bounds__(256) void prep_kernel(const float* C, int k, int d, float* bias,
                                                   uint16_t* Chat, int hf, int8_t* Cq, int u8,
                                                   uint8_t* Cf, const float* sshift,
                                                   float sscale, int sph) {
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= k) return;
  float nrm = 0.0f;
  int nq = 0;  // |q|^2 of the int8 codes, exact
  for (int e = lane; e < d; e += 64) {
    float c = C[(size_t)j * d + e];
    if (Chat) {
      const uint16_t h = to_half_rne(conv_in(c, sshift, sscale, e), hf);
      Chat[(size_t)j * d + e] = h;
      c = half_to_f32(h, hf);
    } else if (Cq) {
      const int8_t q = to_code(c, u8);
      Cq[(size_t)j * d + e] = q;
      nq += (int)q * (int)q;
      continue;
    } else if (Cf) {
      const uint32_t q = f32_to_e4m3(conv_in(c, sshift, sscale, e));
      Cf[(size_t)j * d + e] = (uint8_t)q;
      c = e4m3_to_f32(q);
    }
    nrm += c * c;
  }
  if (Cq) {
    nq = wave_sum(nq);
    if (lane == 0) reinterpret_cast<int32_t*>(bias)[j] = -nq;
    return;
  }
  nrm = wave_sum(nrm);
  if (lane == 0) bias[j] = sph ? 0.0f : -0.5f * nrm;  // spherical: score = x.c
}

// Single workgroup: exclusive scan of the counts (row offsets of the buckets)
// and the list of overflow work items. Work item j < k of the grouping is the
// first R rows of cluster j; a cluster with n > R rows also gets (n - 1) / R
// overflow items, listed here as (cluster, part) pairs. Clusters are taken in
// tiles of 1024 x 16: counts are loaded coalesced (the next tile's loads are
// in flight during this tile's scan) and transposed through LDS so that each
// thread owns 16 consecutive clusters; one block scan of the packed pair (rows
// in the high word, overflow items in the low word) serves both sums, and the
// row offsets go back through LDS to be stored coalesced.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ counts, int k,
                                                    int R, int rsh, int32_t* __restrict__ off,
                                                    int32_t* __restrict__ cursor,
                                                    int2* __restrict__ ovf,
                                                    int32_t* __restrict__ ovf_n,
                                                    int32_t* __restrict__ acc) {
  constexpr int V = 16, kTile = 1024 * V;
  __shared__ int lds[kTile + kTile / 16];
  __shared__ uint64_t tmp[16];
  const auto at = [](int i) { return i + (i >> 4); };  // odd stride: no bank conflicts
  const int tid = threadIdx.x;
  uint64_t carry = 0;
  int nx[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int j = v * 1024 + tid;
    nx[v] = j < k ? counts[j] : 0;
  }
  for (int t0 = 0; t0 < k; t0 += kTile) {
#pragma unroll
    for (int v = 0; v < V; ++v) lds[at(v * 1024 + tid)] = nx[v];
    __syncthreads();
    int n[V];
#pragma unroll
    for (int v = 0; v < V; ++v) n[v] = lds[at(tid * V + v)];
    const int t1 = t0 + kTile;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int j = t1 + v * 1024 + tid;
      nx[v] = j < k ? counts[j] : 0;
    }
    if (acc) {  // the piece's counts join the update's totals and are cleared
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int j = t0 + v * 1024 + tid;
        if (j < k) {
          acc[j] += lds[at(v * 1024 + tid)];
          counts[j] = 0;
        }
      }
    }
    uint64_t loc = 0;
#pragma unroll
    for (int v = 0; v < V; ++v)
      loc += ((uint64_t)(uint32_t)n[v] << 32) | (uint32_t)(n[v] > R ? (n[v] - 1) >> rsh : 0);
    // ends with a barrier: every thread has read its counts from lds
    const uint64_t incl = block_incl_scan<uint64_t, 1024>(loc, tmp);
    const uint64_t total = tmp[15];
    const uint64_t ex = carry + incl - loc;
    int oc = (int)(ex >> 32), ov = (int)(uint32_t)ex;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      lds[at(tid * V + v)] = oc;
      const int extra = n[v] > R ? (n[v] - 1) >> rsh : 0;  // R = 2^rsh
      for (int q = 0; q < extra; ++q) ovf[ov + q] = make_int2(t0 + tid * V + v, q + 1);
      oc += n[v];
      ov += extra;
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int j = t0 + v * 1024 + tid;
      if (j < k) {
        const int o = lds[at(v * 1024 + tid)];
        off[j] = o;
        cursor[j] = o;
      }
    }
    carry += total;
    __syncthreads();  // lds and tmp are rewritten by the next tile
  }
  if (tid == 0) {
    off[k] = (int)(carry >> 32);
    *ovf_n = (int)(uint32_t)carry;
  }
}

// Rows [beg, end) of the bucketed order that work item w sums, the cluster j,
// and whether the cluster is held by this item alone. False for an empty item.
__device__ __forceinline__ bool group_item(int w, int k, int R, const int32_t* __restrict__ off,
                                           const int2* __restrict__ ovf,
                                           const int32_t* __restrict__ ovf_n, int& j, int& beg,
                                           int& end, bool& single) {
  int p = 0;
  if (w < k) {
    j = w;
  } else {
    if (w - k >= *ovf_n) return false;
    const int2 e = ovf[w - k];
    j = e.x;
    p = e.y;
  }
  const int o0 = off[j], o1 = off[j + 1];
  beg = o0 + p * R;
  if (beg >= o1) return false;
  end = min(o1, beg + R);
  single = o1 - o0 <= R;
  return true;
}

// A label outside [0, k) (a row a closing replay leaves out) is not bucketed;
// the counts of launch_label_hist skip the same rows.
__global__ void scatter_kernel(const int32_t* labels, const uint32_t* rows, int nb, int k,
                               int32_t* cursor, uint32_t* order, int2* olab,
                               int32_t* out_labels) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= nb) return;
  const int j = labels[r];
  if ((unsigned)j >= (unsigned)k) return;
  const uint32_t row = rows ? rows[r] : (uint32_t)r;
  const int pos = atomicAdd(&cursor[j], 1);
  order[pos] = row;
  if (olab) olab[pos] = make_int2((int)row, j);
  if (out_labels) out_labels[row] = j;
}

// Counts of the labels a caller supplies (the closing replay): labels in
// [0, k) are counted, -1 marks a row to leave out, and any other value is
// left out too and counted in *bad (reported on the host).
__global__ void label_hist_kernel(const int32_t* __restrict__ labels, int nb, int k,
                                  int32_t* __restrict__ counts, int32_t* __restrict__ bad) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= nb) return;
  const int j = labels[r];
  if ((unsigned)j < (unsigned)k)
    atomicAdd(&counts[j], 1);
  else if (j != -1)
    atomicAdd(bad, 1);
}

// One wave per cluster: the replayed rows' counts and sums join the closing
// statistics (pass_counts, LS); counts and s_acc are reset for the next call.
__global__ __launch_bounds__(256) void closing_add_kernel(int k, int d, int32_t* counts,
                                                          float* s_acc, int32_t* pass_counts,
                                                          float* LS) {
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= k) return;
  const int n = counts[j];
  if (n == 0) return;
  const size_t base = (size_t)j * d;
  for (int e = lane; e < d; e += 64) {
    LS[base + e] += s_acc[base + e];
    s_acc[base + e] = 0.0f;
  }
  if (lane == 0) {
    pass_counts[j] += n;
    counts[j] = 0;
  }
}

// Column unit `col` of a row as fp32 values: 16 bytes of fp32 / bf16 / fp16
// (VEC), 4 bytes of int8, uint8 or E4M3 codes (VEC), or one element.
template <int DT, bool VEC>
__device__ __forceinline__ void load_unit_dt(const unsigned char* base, int col, float* v) {
  if constexpr (VEC && (DT == 2 || DT == 3 || DT == 5)) {
    const uint32_t q = *reinterpret_cast<const uint32_t*>(base + (size_t)col * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (DT == 3)
        v[e] = e4m3_to_f32((q >> (8 * e)) & 0xFFu);
      else if constexpr (DT == 5)
        v[e] = (float)((q >> (8 * e)) & 0xFFu);
      else
        v[e] = (float)(int8_t)(q >> (8 * e));
    }
  } else if constexpr (VEC) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 q = *reinterpret_cast<const u32x4*>(base + (size_t)col * 16);
    if constexpr (DT == 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(q[e] << 16);
        v[2 * e + 1] = __uint_as_float(q[e] & 0xFFFF0000u);
      }
    } else if constexpr (DT == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = f16_to_f32((uint16_t)(q[e] & 0xFFFFu));
        v[2 * e + 1] = f16_to_f32((uint16_t)(q[e] >> 16));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(q[e]);
    }
  } else {
    if constexpr (DT == 1)
      v[0] = bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[col]);
    else if constexpr (DT == 2)
      v[0] = (float)reinterpret_cast<const int8_t*>(base)[col];
    else if constexpr (DT == 3)
      v[0] = e4m3_to_f32(base[col]);
    else if constexpr (DT == 4)
      v[0] = f16_to_f32(reinterpret_cast<const uint16_t*>(base)[col]);
    else if constexpr (DT == 5)
      v[0] = (float)base[col];
    else
      v[0] = reinterpret_cast<const float*>(base)[col];
  }
}

// One workgroup per work item: up to R rows of one cluster (rows taken from
// the bucketed order). Columns are 16-byte chunks when the rows allow it.
// Threads are arranged as rpar row groups x ncol columns (blockDim.x =
// rpar * ncol rounded up to whole waves, at most 256); row groups are folded
// through LDS; a cluster held by a single item is stored, otherwise its
// partial sums are added atomically. Eight row loads are kept in flight per
// thread.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void group_kernel(const unsigned char* __restrict__ X, int d,
                                                    const uint32_t* __restrict__ order,
                                                    const int32_t* __restrict__ off,
                                                    const int2* __restrict__ ovf,
                                                    const int32_t* __restrict__ ovf_n, int k,
                                                    int R, float* __restrict__ s_acc, int add) {
  // element bytes: fp32 4, bf16 / fp16 2, int8 / uint8 / E4M3 1; a column
  // unit is 16 bytes (4 for the 1-byte types, which keeps the rows in flight
  // within the register budget)
  constexpr int ES = DT == 0 ? 4 : (DT == 1 || DT == 4) ? 2 : 1;
  constexpr int UB = ES == 1 ? 4 : 16;
  constexpr int EPV = VEC ? UB / ES : 1;  // elements per column unit
  constexpr int U = 8;                    // rows in flight per thread
  __shared__ float red[256 * EPV];
  int j, beg, end;
  bool single;
  if (!group_item(blockIdx.x, k, R, off, ovf, ovf_n, j, beg, end, single)) return;
  const int tid = threadIdx.x;
  const int NT = blockDim.x;
  const int ncol = d / EPV;
  const size_t rowbytes = (size_t)d * ES;
  float* dst = s_acc + (size_t)j * d;

  auto load_unit = [&](uint32_t row, int col, float* v) {
    const unsigned char* base = X + (size_t)row * rowbytes;
    load_unit_dt<DT, VEC>(base, col, v);
  };


  // sum rows beg+first, beg+first+stride, ... < end of column col into acc
  auto sum_rows = [&](int first, int stride, int col, float* acc) {
    int pos = beg + first;
    for (; pos + (U - 1) * stride < end; pos += U * stride) {
      uint32_t rr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) rr[u] = order[pos + u * stride];
      float v[U][EPV];
#pragma unroll
      for (int u = 0; u < U; ++u) load_unit(rr[u], col, v[u]);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] += v[u][e];
    }
    for (; pos < end; pos += stride) {
      float v[EPV];
      load_unit(order[pos], col, v);
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] += v[e];
    }
  };

  auto write_out = [&](int col, const float* acc) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      if (single && !add)
        dst[col * EPV + e] = acc[e];
      else if (single)
        dst[col * EPV + e] += acc[e];  // later pieces of one update add to the sums
      else
        atomicAdd(&dst[col * EPV + e], acc[e]);
    }
  };

  if (ncol >= NT) {
    for (int col = tid; col < ncol; col += NT) {
      float acc[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;
      sum_rows(0, 1, col, acc);
      write_out(col, acc);
    }
    return;
  }

  const int rpar = NT / ncol;
  const int rg = tid / ncol;
  const int col = tid - rg * ncol;
  float acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;
  if (rg < rpar) {
    sum_rows(rg, rpar, col, acc);
    if (rpar > 1) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) red[(rg * ncol + col) * EPV + e] = acc[e];
    }
  }
  if (rpar > 1) __syncthreads();
  if (rg == 0) {
    for (int g = 1; g < rpar; ++g)
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] += red[(g * ncol + col) * EPV + e];
    write_out(col, acc);
  }
}

// Narrow rows (at most 64 column units of 16 bytes, e.g. d <= 256 fp32 or
// d <= 512 bf16): one wave per work item, four items per workgroup. The 64
// lanes form 64 / ncol row groups; row groups are folded with cross-lane
// shuffles, so a wave needs no LDS and no barrier.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void group_wave_kernel(const unsigned char* __restrict__ X,
                                                         int d, const uint32_t* __restrict__ order,
                                                         const int32_t* __restrict__ off,
                                                         const int2* __restrict__ ovf,
                                                         const int32_t* __restrict__ ovf_n,
                                                         int k, int R, float* __restrict__ s_acc,
                                                         int add) {
  // element bytes: fp32 4, bf16 / fp16 2, int8 / uint8 / E4M3 1; a column
  // unit is 16 bytes (4 for the 1-byte types, which keeps the rows in flight
  // within the register budget)
  constexpr int ES = DT == 0 ? 4 : (DT == 1 || DT == 4) ? 2 : 1;
  constexpr int UB = ES == 1 ? 4 : 16;
  constexpr int EPV = VEC ? UB / ES : 1;  // elements per column unit
  constexpr int U = 8;                    // rows in flight per lane
  const int lane = threadIdx.x & 63;
  int j, beg, end;
  bool single;
  if (!group_item(blockIdx.x * 4 + (threadIdx.x >> 6), k, R, off, ovf, ovf_n, j, beg, end, single))
    return;
  const int ncol = d / EPV;
  const int rpar = 64 / ncol;
  const int rg = lane / ncol;
  const int col = lane - rg * ncol;
  const size_t rowbytes = (size_t)d * ES;

  auto load_unit = [&](uint32_t row, float* v) {
    const unsigned char* base = X + (size_t)row * rowbytes;
    load_unit_dt<DT, VEC>(base, col, v);
  };

  float acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;
  if (rg < rpar) {
    int pos = beg + rg;
    for (; pos + (U - 1) * rpar < end; pos += U * rpar) {
      uint32_t rr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) rr[u] = order[pos + u * rpar];
      float v[U][EPV];
#pragma unroll
      for (int u = 0; u < U; ++u) load_unit(rr[u], v[u]);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] += v[u][e];
    }
    for (; pos < end; pos += rpar) {
      float v[EPV];
      load_unit(order[pos], v);
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] += v[e];
    }
  }
  // fold the row groups into row group 0 (lanes 0 .. ncol-1)
  for (int g = 1; g < rpar; ++g) {
    const int src = col + g * ncol;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const float o = __shfl(acc[e], src, 64);
      if (rg == 0) acc[e] += o;
    }
  }
  if (rg == 0) {
    float* dst = s_acc + (size_t)j * d + (size_t)col * EPV;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      if (single && !add)
        dst[e] = acc[e];
      else if (single)
        dst[e] += acc[e];  // later pieces of one update add to the sums
      else
        atomicAdd(&dst[e], acc[e]);
    }
  }
}

// UB raw bytes of a row (UB = 4, 8 or 16) into UB / 4 dwords, and their
// values as fp32 (fp32, bf16, fp16, int8 codes, E4M3 codes or uint8 values).
// Split so that a batch of row loads is issued before any of them is
// converted.
// The rows are read once per step: non-temporal loads, which keep the
// gathered rows from displacing the rest of L2 (the 4M-row bf16 batches:
// 255 -> 208 us per grouping launch; the deep- and SIFT-like batches about
// 1.5% faster).
template <int UB>
__device__ __forceinline__ void load_unit_raw(const unsigned char* p, uint32_t* r) {
#pragma unroll
  for (int e = 0; e < UB / 4; ++e)
    r[e] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p) + e);
}

template <int DT, int UB>
__device__ __forceinline__ void unit_to_f32(const uint32_t* r, float* v) {
#pragma unroll
  for (int h = 0; h < UB / 4; ++h) {
    const uint32_t q = r[h];
    if constexpr (DT == 2 || DT == 3 || DT == 5) {  // 1-byte codes / values
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t b = (q >> (8 * e)) & 0xFFu;
        if constexpr (DT == 3)
          v[4 * h + e] = e4m3_to_f32(b);
        else if constexpr (DT == 5)
          v[4 * h + e] = (float)b;
        else
          v[4 * h + e] = (float)(int8_t)b;
      }
    } else if constexpr (DT == 1) {  // bf16
      v[2 * h] = __uint_as_float(q << 16);
      v[2 * h + 1] = __uint_as_float(q & 0xFFFF0000u);
    } else if constexpr (DT == 4) {  // fp16
      v[2 * h] = f16_to_f32((uint16_t)(q & 0xFFFFu));
      v[2 * h + 1] = f16_to_f32((uint16_t)(q >> 16));
    } else {  // fp32
      v[h] = __uint_as_float(q);
    }
  }
}

// Grouping of narrow rows (a row is at most 64 units of UB bytes): one wave
// per span of C consecutive clusters, whose rows occupy one contiguous run of
// the bucketed order. Each lane owns one UB-byte column unit of every row.
// The wave reads the span's C + 1 offsets in one load and the run's row ids in
// 64-slot chunks (one load each), then issues the row loads U at a time,
// summing in slot order and storing each cluster's sum when its last slot
// has been added, so the dependent chain per wave is offsets -> row ids ->
// rows however many clusters the span holds. A span holding a cluster of
// more than R rows (rare for the mixtures these rows come from) takes the
// per-cluster path: part 0 of each cluster here, parts >= 1 as the overflow
// items that follow the spans (waves nA and up), with atomic adds for
// clusters split over items. Without `add` the sums are stored (s_acc of a
// cluster with rows need not be zero); with `add` (a later piece of one
// update) every span takes the per-cluster path and adds them. U row loads
// are in flight per lane: 16 for spans of a few short clusters, 32 where a
// span is one cluster of tens of rows (fewer dependent rounds per wave).
template <int DT, int UB, int U = 16>
__global__ __launch_bounds__(256) void group_span_kernel(const unsigned char* __restrict__ X,
                                                         int d, const uint32_t* __restrict__ order,
                                                         const int32_t* __restrict__ off,
                                                         const int2* __restrict__ ovf,
                                                         const int32_t* __restrict__ ovf_n,
                                                         int k, int R, int C, int nA,
                                                         float* __restrict__ s_acc, int add) {
  constexpr int ES = DT == 0 ? 4 : (DT == 1 || DT == 4) ? 2 : 1;
  constexpr int EPV = UB / ES;  // elements per lane per row
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t rowbytes = (size_t)d * ES;
  const int ncol = (int)(rowbytes / UB);
  const bool active = lane < ncol;
  // idle lanes read their row's first unit (a valid address; never stored),
  // so the loads below need no lane mask and stay in flight together
  const unsigned char* xcol = X + (active ? (size_t)lane * UB : 0);

  float acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;

  auto flush = [&](int j, bool single) {
    if (active) {
      float* dst = s_acc + (size_t)j * d + (size_t)lane * EPV;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        if (single && !add)
          dst[e] = acc[e];
        else if (single)
          dst[e] += acc[e];
        else
          atomicAdd(&dst[e], acc[e]);
        acc[e] = 0.0f;
      }
    }
  };

  // slots [beg, end) of the order, all of cluster j, into acc
  auto sum_run = [&](int beg, int end) {
    for (int t = beg; t < end; t += 64) {
      const int m = min(64, end - t);
      const int ord = lane < m ? (int)order[t + lane] : 0;
      for (int u = 0; u < m; u += U) {
        uint32_t raw[U][UB / 4];
#pragma unroll
        for (int q = 0; q < U; ++q) {  // slots past m re-read the last row (not added)
          const uint32_t row = (uint32_t)__builtin_amdgcn_readlane(ord, min(u + q, m - 1));
          load_unit_raw<UB>(xcol + (size_t)row * rowbytes, raw[q]);
        }
#pragma unroll
        for (int q = 0; q < U; ++q)
          if (u + q < m) {
            float v[EPV];
            unit_to_f32<DT, UB>(raw[q], v);
#pragma unroll
            for (int e = 0; e < EPV; ++e) acc[e] += v[e];
          }
      }
    }
  };

  if (w >= nA) {  // overflow item: part p >= 1 of a cluster of more than R rows
    const int it = w - nA;
    if (it >= *ovf_n) return;
    const int2 o = ovf[it];
    const int b = off[o.x], e = off[o.x + 1];
    const int beg = b + o.y * R;
    if (beg >= e) return;
    sum_run(beg, min(e, beg + R));
    flush(o.x, false);
    return;
  }

  const int j0 = w * C;
  const int nc = min(C, k - j0);
  const int my_off = lane <= nc ? off[j0 + lane] : 0;
  const int nxt = __shfl_down(my_off, 1, 64);
  const bool big = lane < nc && nxt - my_off > R;
  // per cluster (part 0 of each, atomics where split) when the span holds a
  // cluster of more than R rows or the sums are added to earlier pieces
  if (add || __ballot(big) != 0ull) {
    for (int jj = 0; jj < nc; ++jj) {
      const int b = __builtin_amdgcn_readlane(my_off, jj);
      const int e = __builtin_amdgcn_readlane(my_off, jj + 1);
      if (b == e) continue;
      sum_run(b, min(e, b + R));
      flush(j0 + jj, e - b <= R);
    }
    return;
  }

  // the span's slots in order, each cluster stored when its last slot is in
  const int S0 = __builtin_amdgcn_readlane(my_off, 0);
  const int S1 = __builtin_amdgcn_readlane(my_off, nc);
  int jc = 0;  // current cluster (relative to j0); its rows end at bnd
  int bnd = __builtin_amdgcn_readlane(my_off, 1);
  while (bnd == S0 && jc + 1 < nc) bnd = __builtin_amdgcn_readlane(my_off, ++jc + 1);
  for (int t = S0; t < S1; t += 64) {
    const int m = min(64, S1 - t);
    const int ord = lane < m ? (int)order[t + lane] : 0;
    for (int u = 0; u < m; u += U) {
      uint32_t raw[U][UB / 4];
#pragma unroll
      for (int q = 0; q < U; ++q) {  // slots past m re-read the last row (not added)
        const uint32_t row = (uint32_t)__builtin_amdgcn_readlane(ord, min(u + q, m - 1));
        load_unit_raw<UB>(xcol + (size_t)row * rowbytes, raw[q]);
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        if (u + q < m) {
          float v[EPV];
          unit_to_f32<DT, UB>(raw[q], v);
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[e] += v[e];
          const int slot = t + u + q;
          if (slot + 1 == bnd) {  // last row of cluster jc: store, move to the next with rows
            if (active) {
              float* dst = s_acc + (size_t)(j0 + jc) * d + (size_t)lane * EPV;
#pragma unroll
              for (int e = 0; e < EPV; ++e) {
                dst[e] = acc[e];
                acc[e] = 0.0f;
              }
            }
            do {
              ++jc;
              bnd = jc < nc ? __builtin_amdgcn_readlane(my_off, jc + 1) : 0x7FFFFFFF;
            } while (bnd == slot + 1);
          }
        }
      }
    }
  }
}

// Grouping of narrow rows by windows of the bucketed order, for batches of
// small clusters (a few rows each on average). Wave w owns the clusters whose
// first slot lies in [W w, W w + W). It reads the (row id, label) pairs of
// slots W w .. W w + 63, one 8-byte load per lane (lanes W..63 are a
// look-ahead that normally holds the rest of its last cluster; the label of
// the slot before each lane's comes from a lane shift), then the rows of its
// clusters, U loads in flight per lane, so its dependent chain is
// labels -> rows -> stores (the span kernel's read of the cluster offsets is
// gone). Each cluster with rows is summed by exactly one wave, in slot order,
// and stored (added with `add`); a last cluster that runs past the look-ahead
// is finished in further 64-slot chunks. Each lane owns one UB-byte column
// unit of every row. Slots past the owned ones in a batch of U loads re-read
// the last owned row (a cache hit, not added), so the loads need no branch.
template <int DT, int UB, int U, int W>
__global__ __launch_bounds__(256) void group_win_kernel(const unsigned char* __restrict__ X,
                                                        int d, const int2* __restrict__ olab,
                                                        const int32_t* __restrict__ off, int k,
                                                        int nb, float* __restrict__ s_acc,
                                                        int add) {
  constexpr int ES = DT == 0 ? 4 : (DT == 1 || DT == 4) ? 2 : 1;
  constexpr int EPV = UB / ES;  // elements per lane per row
  constexpr int RW = UB / 4;    // dwords per lane per row
  const int lane = threadIdx.x & 63;
  const int s0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * W;
  if (s0 >= nb) return;
  const size_t rowbytes = (size_t)d * ES;
  const int ncol = (int)(rowbytes / UB);
  const bool active = lane < ncol;
  const unsigned char* xcol = X + (active ? (size_t)lane * UB : 0);

  // one round of independent loads: this lane's slot, the slot before it, and
  // the number of bucketed slots (addresses clamped into the nb-slot buffers;
  // slots at or past ns are masked below)
  const int sl = s0 + lane;
  const int sc = min(sl, nb - 1);
  const int2 pr = olab[sc];
  const int lab = pr.y;
  const uint32_t ord = (uint32_t)pr.x;
  const int lab0 = olab[max(s0 - 1, 0)].y;  // the slot before the window
  const int ns = off[k];
  // label of the slot before this lane's: lane - 1's (wave_shr:1), lab0 on lane 0
  const int labp = __builtin_amdgcn_update_dpp(lab0, lab, 0x138, 0xF, 0xF, false);
  const bool valid = sl < ns;
  const bool start = valid && (sl == 0 || lab != labp);
  const uint64_t own = __ballot(start && lane < W);
  if (own == 0ull) return;  // the window lies inside a cluster that began earlier
  // the owned slots are lanes [a, e): e is the first slot past the end of the
  // bucketed order or the first cluster start in the look-ahead
  const uint64_t endm = __ballot(!valid || (lane >= W && start));
  const int a = __builtin_ctzll(own);
  const int e = endm ? __builtin_ctzll(endm) : 64;

  float acc[EPV];
#pragma unroll
  for (int q = 0; q < EPV; ++q) acc[q] = 0.0f;
  auto flush = [&](int j) {
    if (active) {
      float* dst = s_acc + (size_t)j * d + (size_t)lane * EPV;
      if (add) {
#pragma unroll
        for (int q = 0; q < EPV; ++q) dst[q] += acc[q];
      } else if constexpr (EPV % 4 == 0) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int q = 0; q < EPV; q += 4)
          *reinterpret_cast<f32x4*>(dst + q) = f32x4{acc[q], acc[q + 1], acc[q + 2], acc[q + 3]};
      } else if constexpr (EPV == 2) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<f32x2*>(dst) = f32x2{acc[0], acc[1]};
      } else {
        dst[0] = acc[0];
      }
    }
#pragma unroll
    for (int q = 0; q < EPV; ++q) acc[q] = 0.0f;
  };

  for (int t = a; t < e; t += U) {
    uint32_t raw[U][RW];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const uint32_t row = (uint32_t)__builtin_amdgcn_readlane((int)ord, min(t + q, e - 1));
      load_unit_raw<UB>(xcol + (size_t)row * rowbytes, raw[q]);
    }
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int sq = t + q;
      if (sq < e) {
        float v[EPV];
        unit_to_f32<DT, UB>(raw[q], v);
#pragma unroll
        for (int c = 0; c < EPV; ++c) acc[c] += v[c];
        // a cluster ends at slot sq when the next slot holds another label,
        // or at e unless e is the end of the look-ahead (the cluster goes on)
        const int lq = __builtin_amdgcn_readlane(lab, sq);
        const bool last = sq + 1 < e ? __builtin_amdgcn_readlane(lab, sq + 1) != lq : e < 64;
        if (last) flush(lq);
      }
    }
  }
  if (e < 64) return;
  // the last cluster runs past the look-ahead: its rows in 64-slot chunks
  const int lc = __builtin_amdgcn_readlane(lab, 63);
  for (int t0 = s0 + 64;; t0 += 64) {
    const int sl2 = t0 + lane;
    const int sc2 = min(sl2, nb - 1);
    const int2 pr2 = olab[sc2];
    const int lab2 = pr2.y;
    const uint32_t ord2 = (uint32_t)pr2.x;
    const uint64_t stop = __ballot(sl2 >= ns || lab2 != lc);
    const int m = stop ? __builtin_ctzll(stop) : 64;
    for (int t = 0; t < m; t += U) {
      uint32_t raw[U][RW];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const uint32_t row = (uint32_t)__builtin_amdgcn_readlane((int)ord2, min(t + q, m - 1));
        load_unit_raw<UB>(xcol + (size_t)row * rowbytes, raw[q]);
      }
#pragma unroll
      for (int q = 0; q < U; ++q)
        if (t + q < m) {
          float v[EPV];
          unit_to_f32<DT, UB>(raw[q], v);
#pragma unroll
          for (int c = 0; c < EPV; ++c) acc[c] += v[c];
        }
    }
    if (m < 64) break;
  }
  flush(lc);
}

// One wave per cluster: EMA of the running count and sum, centroid S/N,
// search-format refresh, last-pass accumulation; resets counts and s_acc.
// search format kept beside C: 0 none, 1 bf16 (Chat), 2 int8 (Cq), 3 E4M3 (Cf),
// 4 fp16 (Chat), 5 shifted uint8 (Cq)
template <int SF>
__global__ __launch_bounds__(256) void ema_kernel(int k, int d, float a, float b,
                                                  int32_t* __restrict__ counts,
                                                  float* __restrict__ s_acc, float* __restrict__ N,
                                                  float* __restrict__ S, float* __restrict__ C,
                                                  float* __restrict__ bias,
                                                  uint16_t* __restrict__ Chat,
                                                  int8_t* __restrict__ Cq, uint8_t* __restrict__ Cf,
                                                  int32_t* __restrict__ pass_counts,
                                                  float* __restrict__ LS, int sph, float beta,
                                                  float b2, float* __restrict__ N2,
                                                  float* __restrict__ S2,
                                                  const float* __restrict__ sshift, float sscale) {
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= k) return;
  const int n = counts[j];
  const float Nn = __fadd_rn(__fmul_rn(b, N[j]), __fmul_rn(a, (float)n));
  float nrm = 0.0f;
  int nq = 0;  // |q|^2 of the int8 codes, exact
  const size_t base = (size_t)j * d;
  // G elements per lane at a time: all their loads first, then the
  // arithmetic and the stores, so that a wave waits for memory once per G
  // elements instead of once per element
  constexpr int G = 8;
  for (int e0 = lane; e0 < d; e0 += 64 * G) {
    float sv[G], Sv[G], S2v[G], Cv[G], LSv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int e = e0 + 64 * g;
      sv[g] = 0.0f;
      S2v[g] = Cv[g] = LSv[g] = 0.0f;
      Sv[g] = 0.0f;
      if (e < d) {
        const size_t idx = base + e;
        if (n) sv[g] = s_acc[idx];
        Sv[g] = S[idx];
        if (S2) S2v[g] = S2[idx];
        if (!(Nn > 0.0f)) Cv[g] = C[idx];
        if (LS && n) LSv[g] = LS[idx];
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int e = e0 + 64 * g;
      if (e >= d) continue;
      const size_t idx = base + e;
      const float s = sv[g];
      if (n) s_acc[idx] = 0.0f;
      const float Snew = __fadd_rn(__fmul_rn(b, Sv[g]), __fmul_rn(a, s));
      S[idx] = Snew;
      if (S2) S2[idx] = __fadd_rn(__fmul_rn(b2, S2v[g]), __fmul_rn(beta, s));
      float c;
      if (Nn > 0.0f) {
        c = __fdiv_rn(Snew, Nn);
        C[idx] = c;
      } else {
        c = Cv[g];
      }
      if (LS && n) LS[idx] = LSv[g] + s;
      if (sph) continue;  // rescaled (and rounded to Chat) below, once the norm is known
      if constexpr (SF == 1 || SF == 4) {
        const uint16_t h = to_half_rne(conv_in(c, sshift, sscale, e), SF == 4);
        Chat[idx] = h;
        c = half_to_f32(h, SF == 4);
      } else if constexpr (SF == 2 || SF == 5) {
        const int8_t q = to_code(c, SF == 5);
        Cq[idx] = q;
        nq += (int)q * (int)q;
        continue;
      } else if constexpr (SF == 3) {
        const uint32_t q = f32_to_e4m3(conv_in(c, sshift, sscale, e));
        Cf[idx] = (uint8_t)q;
        c = e4m3_to_f32(q);
      }
      nrm += c * c;
    }
  }
  if constexpr (SF == 2 || SF == 5) nq = wave_sum(nq);
  if (sph) {
    // spherical e-means: S / N rescaled to norm 1 (a centroid without a
    // count keeps its unit-norm value); the score is x.c, bias 0
    if (Nn > 0.0f) wave_normalize(C + base, d, lane);
    if constexpr (SF == 1 || SF == 4)
      for (int e = lane; e < d; e += 64) Chat[base + e] = to_half_rne(C[base + e], SF == 4);
  } else {
    nrm = wave_sum(nrm);
  }
  if (lane == 0) {
    N[j] = Nn;
    if (N2) N2[j] = __fadd_rn(__fmul_rn(b2, N2[j]), __fmul_rn(beta, (float)n));
    if constexpr (SF == 2 || SF == 5)
      reinterpret_cast<int32_t*>(bias)[j] = -nq;
    else
      bias[j] = sph ? 0.0f : -0.5f * nrm;
    pass_counts[j] += n;
    counts[j] = 0;
  }
}

// One wave per centroid: the slow centroids S2 / N2 (C where N2 = 0, or
// everywhere without a slow pair), rescaled to norm 1 with sph.
__global__ __launch_bounds__(256) void slow_final_kernel(int k, int d, const float* N2,
                                                         const float* S2, const float* C,
                                                         float* out, int sph) {
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= k) return;
  const float nn = N2 ? N2[j] : 0.0f;
  const size_t base = (size_t)j * d;
  for (int e = lane; e < d; e += 64)
    out[base + e] = nn > 0.0f ? __fdiv_rn(S2[base + e], nn) : C[base + e];
  if (sph && nn > 0.0f) wave_normalize(out + base, d, lane);
}

// Dead-cluster revival. Mean running count m = sum N / k (fp64); dead set
// D = {j : N_j < thr * m} in index order (Lloyd's empty-cluster split:
// D = {j : N_j = 0}, the counts being whole numbers). For each dead j in turn: u from
// Philox, donor i = first live index whose fp64 prefix sum of N over live
// clusters exceeds u * (sum of live N); the donor keeps half of its count and
// sum, cluster j takes the other half, and both sums are perturbed by
// -/+ 2^-10 * sign per coordinate.
//
// Up to k = 16384, revive_spec_kernel (below) draws the donors; beyond it
// revive_kernel (one workgroup):
//  A. all threads: threshold, dead list, uniform draws, live counts (in LDS
//     when k <= kRvLdsN), fp64 live sum of each of 64 chunks of CS = 64 V
//     consecutive clusters.
//  B. wave 0 alone draws the donors in dead-list order. Lane c owns chunk c
//     and keeps its live sum and the inclusive prefix of the sums over lanes
//     in registers. A draw finds the chunk with one ballot, then reads the
//     chunk's live counts (V consecutive clusters per lane), takes the lane's
//     running sums in registers plus one wave scan, and finds the cluster with
//     a second ballot; then it subtracts the donor's lost half from the
//     prefixes. Only running counts change here.
//  C. all threads: chain bookkeeping. A donor picked r times before split q
//     had its count halved r times, so the recorded count after split q fixes
//     q's place in the donor's chain and the final count the chain's length.
// Both end with the same chain bookkeeping (revive_chains), and then
// split_kernel (many workgroups): one wave per chain applies its splits of the
// running sums in order (chains are independent: donors are never dead).
constexpr int kRvLdsN = 32768;  // live counts kept in LDS up to this k

__device__ __forceinline__ int halvings(float from, float to) {
  int m = 0;
  while (from != to && m < 200) {
    from *= 0.5f;
    ++m;
  }
  return m;
}

// Chain bookkeeping after the draws (all 1024 threads of the revival
// workgroup): a donor picked r times before split q had its count halved r
// times, so the recorded count after split q fixes q's place in the donor's
// chain and the final count the chain's length. Per thread a contiguous run
// of splits; chain starts are counted with a block scan (chain lengths) and a
// second one (number of chains).
__device__ __forceinline__ void revive_chains(const ReviveArgs& A, int ndead, int* itmp) {
  constexpr int G = 8;  // splits per batch: their loads are issued together
  const int tid = threadIdx.x;
  const int qper = (ndead + 1023) / 1024;
  const int q0 = min(ndead, tid * qper), q1 = min(ndead, q0 + qper);
  int lensum = 0, hcnt = 0;
  for (int qb = q0; qb < q1; qb += G) {
    int iv[G];
    float pn[G], n0v[G], nfv[G];
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const int q = min(qb + e, q1 - 1);
      iv[e] = A.pair_i[q];
      pn[e] = A.pair_n[q];
    }
#pragma unroll
    for (int e = 0; e < G; ++e) {
      n0v[e] = A.n0[iv[e]];
      nfv[e] = A.N[iv[e]];
    }
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const int q = qb + e;
      if (q < q1) {
        const int ps = halvings(n0v[e] * 0.5f, pn[e]);
        A.pos[q] = ps;
        if (ps == 0) {
          const int len = 1 + halvings(n0v[e] * 0.5f, nfv[e]);
          A.head_of[iv[e]] = q;
          A.clen[q] = len;
          lensum += len;
          ++hcnt;
        }
      }
    }
  }
  const int lincl = block_incl_scan<int, 1024>(lensum, itmp);
  const int hincl = block_incl_scan<int, 1024>(hcnt, itmp);
  int lb = lincl - lensum, hb = hincl - hcnt;
  for (int qb = q0; qb < q1; qb += G) {
    int pv[G], cl[G];
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const int q = min(qb + e, q1 - 1);
      pv[e] = A.pos[q];
      cl[e] = A.clen[q];
    }
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const int q = qb + e;
      if (q < q1 && pv[e] == 0) {
        A.cbase[q] = lb;
        lb += cl[e];
        A.heads[hb++] = q;
      }
    }
  }
  if (tid == 1023) A.nheads[0] = hincl;
  __threadfence_block();
  __syncthreads();
  for (int qb = q0; qb < q1; qb += G) {
    int iv[G], pv[G], hv[G], cb[G];
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const int q = min(qb + e, q1 - 1);
      iv[e] = A.pair_i[q];
      pv[e] = A.pos[q];
    }
#pragma unroll
    for (int e = 0; e < G; ++e) hv[e] = A.head_of[iv[e]];
#pragma unroll
    for (int e = 0; e < G; ++e) cb[e] = A.cbase[hv[e]];
#pragma unroll
    for (int e = 0; e < G; ++e)
      if (qb + e < q1) A.list[cb[e] + pv[e]] = qb + e;
  }
  if (tid == 0) {
    A.counters[0] += ndead;
    A.counters[3] += ndead;
  }
}

// VT > 0: VT clusters per lane per chunk (a power of two >= k / 4096), held in
// registers during a draw; VT = 0: any k, counts re-read.
template <int VT>
__global__ __launch_bounds__(1024) void revive_kernel(ReviveArgs A) {
  __shared__ double dtmp[16];
  __shared__ int itmp[16];
  __shared__ double csum[64];
  // live counts in LDS exactly when VT <= 8 (k <= 32768); a compile-time
  // choice keeps global loads, and waits on the draw's global stores, out of
  // the LDS variant's draw loop
  constexpr bool lds_n = VT >= 1 && VT <= 8;
  __shared__ __attribute__((aligned(16))) float wN[lds_n ? 4096 * VT : 4];
  __shared__ int s_ndead, s_last;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int k = A.k;
  static_assert(8 * 4096 <= kRvLdsN, "VT <= 8 must fit the LDS counts");
  const int V = VT > 0 ? VT : (k + 4095) / 4096;  // clusters per lane per chunk
  const int CS = 64 * V;  // clusters per chunk; chunk c = [c CS, (c + 1) CS)
  if (tid == 0) A.nheads[0] = 0;

  // ---- A --------------------------------------------------------------------
  double loc = 0.0;
  for (int j = tid; j < k; j += 1024) loc += (double)A.N[j];
  const double total = block_sum<double, 1024>(loc, dtmp);
  const double th = A.empty_only ? 0.5 : A.thr * (total / (double)k);

  const int per = (k + 1023) / 1024;
  const int j0 = min(k, tid * per), j1 = min(k, j0 + per);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) {
    const float nv = A.N[j];
    const int dd = ((double)nv < th) ? 1 : 0;
    A.flags[j] = dd;
    A.n0[j] = nv;
    if constexpr (lds_n)
      wN[j] = dd ? 0.0f : nv;
    else
      A.wlive[j] = dd ? 0.0f : nv;  // live counts, read by the draws with wide loads
    cnt += dd;
  }
  // zero counts past k up to the 64 chunks: no bounds test in a draw
  if constexpr (lds_n)
    for (int j = k + tid; j < 64 * CS; j += 1024) wN[j] = 0.0f;
  else if constexpr (VT > 0)
    for (int j = k + tid; j < 64 * CS; j += 1024) A.wlive[j] = 0.0f;
  const int incl = block_incl_scan<int, 1024>(cnt, itmp);
  if (tid == 1023) s_ndead = incl;
  if (tid == 0) s_last = -1;
  int wpos = incl - cnt;
  int mylast = -1;
  for (int j = j0; j < j1; ++j) {
    if (A.flags[j])
      A.dead[wpos++] = j;
    else
      mylast = j;
  }
  __threadfence_block();
  __syncthreads();
  if (mylast >= 0) atomicMax(&s_last, mylast);
  const int ndead = s_ndead;
  if (A.count_only) {
    if (tid == 0) A.counters[2] = ndead;
    return;
  }
  if (ndead == 0) return;
  for (int q = tid; q < ndead; q += 1024)
    A.udraw[q] = revive_uniform(A.seed, A.step, (uint64_t)A.dead[q]);
  {
    // live sum of chunk c by the 16 consecutive threads 16 c .. 16 c + 15
    const int c = tid >> 4, part = tid & 15;
    double sv = 0.0;
    const int e1 = min(k, (c + 1) * CS);
    for (int j = c * CS + part; j < e1; j += 16)
      if (!A.flags[j]) sv += (double)A.N[j];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) sv += __shfl_xor(sv, o, 64);
    if (part == 0) csum[c] = sv;
  }
  __threadfence_block();
  __syncthreads();
  const int last_live = s_last;
  if (last_live < 0) return;  // no donor exists (every cluster under the threshold)

  // ---- B: donor draws (wave 0) ----------------------------------------------
  if (wave == 0) {
    auto live_count = [&](int idx) -> float {
      if constexpr (lds_n) return wN[idx];
      if (idx >= k) return 0.0f;
      return A.wlive[idx];
    };
    double lsum = csum[lane];
    double incA = wave_scan_f64(lsum);
    double T = readlane_f64(incA, 63);
    int64_t logc = A.counters[1];
    int dl = 0;
    double ul = 0.0;
    // With the counts in LDS the draws of a batch of 64 touch no global
    // memory: lane ql keeps draw ql's donor and count, and one coalesced
    // flush per batch writes them (vector stores and loads share one
    // completion counter, so a store inside the loop would make the next
    // batch load wait for it, once per draw).
    int bi = 0;
    float bn = 0.0f;
    for (int q = 0; q < ndead; ++q) {
      const int ql = q & 63;
      if (ql == 0) {
        dl = (q + lane < ndead) ? A.dead[q + lane] : 0;
        ul = (q + lane < ndead) ? A.udraw[q + lane] : 0.0;
      }
      const int j = __builtin_amdgcn_readlane(dl, ql);
      const double target = readlane_f64(ul, ql) * T;
      int donor = -1;
      float nvd = 0.0f;
      const uint64_t bA = __ballot(lsum > 0.0 && incA > target);
      if (bA) {
        const int L = __ffsll((unsigned long long)bA) - 1;
        const double base = readlane_f64(incA - lsum, L);
        const int i0 = L * CS + lane * V;  // this lane's clusters of chunk L
        int vl = -1;                        // this lane's first cluster past the target
        double lp = 0.0;
        float wl = 0.0f;
        if constexpr (VT > 0) {
          float w[VT];
          double pv[VT];
          if constexpr (lds_n) {
            // VT consecutive counts, VT-aligned: one wide LDS read
#pragma unroll
            for (int v = 0; v < VT; v += (VT >= 4 ? 4 : VT)) {
              if constexpr (VT >= 4) {
                const float4 q4 = *reinterpret_cast<const float4*>(&wN[i0 + v]);
                w[v] = q4.x;
                w[v + 1] = q4.y;
                w[v + 2] = q4.z;
                w[v + 3] = q4.w;
              } else if constexpr (VT == 2) {
                const float2 q2 = *reinterpret_cast<const float2*>(&wN[i0 + v]);
                w[v] = q2.x;
                w[v + 1] = q2.y;
              } else {
                w[v] = wN[i0 + v];
              }
            }
          } else {
            // VT consecutive live counts (zero-padded to 64 chunks): independent wide loads
#pragma unroll
            for (int v = 0; v < VT; v += 4) {
              const float4 q4 = *reinterpret_cast<const float4*>(&A.wlive[i0 + v]);
              w[v] = q4.x;
              w[v + 1] = q4.y;
              w[v + 2] = q4.z;
              w[v + 3] = q4.w;
            }
          }
#pragma unroll
          for (int v = 0; v < VT; ++v) {
            lp += (double)w[v];
            pv[v] = lp;
          }
          const double ex = base + wave_scan_f64(lp) - lp;
#pragma unroll
          for (int v = VT - 1; v >= 0; --v)
            if (w[v] > 0.0f && ex + pv[v] > target) {
              vl = v;
              wl = w[v];
            }
        } else {
          for (int v = 0; v < V; ++v) lp += (double)live_count(i0 + v);
          double run = base + wave_scan_f64(lp) - lp;
          for (int v = 0; v < V && vl < 0; ++v) {
            const float wv = live_count(i0 + v);
            run += (double)wv;
            if (wv > 0.0f && run > target) {
              vl = v;
              wl = wv;
            }
          }
        }
        const uint64_t b2 = __ballot(vl >= 0);
        if (b2) {
          const int t2 = __ffsll((unsigned long long)b2) - 1;
          donor = L * CS + t2 * V + __builtin_amdgcn_readlane(vl, t2);
          nvd = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), t2));
        }
      }
      if (donor < 0) {
        donor = last_live;
        if constexpr (lds_n)
          nvd = wN[donor];
        else
          nvd = A.wlive[donor];
      }
      const int i = donor;
      const float Nh = nvd * 0.5f;
      if constexpr (lds_n) {
        if (lane == 0) wN[i] = Nh;
        if (lane == ql) {
          bi = i;
          bn = Nh;
        }
        if (ql == 63 || q + 1 == ndead) {
          // flush draws q - ql .. q: lane l holds draw q - ql + l (dead cluster dl)
          const int q0 = q - ql;
          if (lane <= ql) {
            A.N[dl] = bn;
            A.pair_i[q0 + lane] = bi;
            A.pair_n[q0 + lane] = bn;
            if (A.log && logc + lane < A.log_cap) {
              A.log[3 * (logc + lane)] = (int32_t)A.step;
              A.log[3 * (logc + lane) + 1] = dl;
              A.log[3 * (logc + lane) + 2] = bi;
            }
          }
          if (A.log) logc = min(A.log_cap, logc + ql + 1);
        }
      } else {
        if (lane == 0) {
          A.N[i] = Nh;
          A.N[j] = Nh;
          A.pair_i[q] = i;
          A.pair_n[q] = Nh;
          A.wlive[i] = Nh;
          if (A.log && logc < A.log_cap) {
            A.log[3 * logc] = (int32_t)A.step;
            A.log[3 * logc + 1] = j;
            A.log[3 * logc + 2] = i;
            ++logc;
          }
        }
        // counts read from global memory by the next draw must see these stores
        __threadfence_block();
      }
      // the donor's chunk lost Nh of live count: update the prefix state
      const int Lo = i / CS;
      if (lane == Lo) lsum -= (double)Nh;
      if (lane >= Lo) incA -= (double)Nh;
      T -= (double)Nh;
    }
    if (lane == 0) A.counters[1] = logc;
  }
  __threadfence_block();
  __syncthreads();
  if constexpr (lds_n) {
    // the donors' halved counts, from LDS (dead clusters were written by the flushes)
    for (int j = tid; j < k; j += 1024)
      if (!A.flags[j]) A.N[j] = wN[j];
    __threadfence_block();
    __syncthreads();
  }

  // ---- C: chain bookkeeping -------------------------------------------------
  revive_chains(A, ndead, itmp);
}

// Donor draws for k <= kSpecK, speculated a round of kSpecRound at a time.
//
// The draws are sequential (each halves its donor's count, which moves every
// later target and prefix sum), but one draw moves them little: the donor of
// draw q is usually at or next to the cluster it would get from the counts at
// the start of its round. So each round of kSpecRound dead clusters (lane q = draw q)
//  1. speculates in parallel: lane q searches the round-start prefix sums for
//     u_q T (T = the live total at the round's start) and keeps its candidate
//     m_q with the exact current prefix sums around it, L_q = cum(m_q - 1)
//     and H_q = cum(m_q), and the candidate's current count;
//  2. settles the draws in order: draw q's exact target is u_q T_q (T_q =
//     the live total after the round's earlier draws); if L_q <= u_q T_q <
//     H_q the candidate is the donor (the first cluster whose prefix sum
//     exceeds the target); otherwise a walk from m_q over the current counts,
//     16 clusters per step, finds it. Each settled draw halves its donor's
//     count, and every lane subtracts the lost half from L, H (where the donor
//     lies at or before its candidate) and from T;
//  3. folds the round's halvings into the prefix tree.
// Live clusters are compacted in index order (dead ones carry no weight), and
// the prefix sums come from a tree of sums of 8 (levels of 2048, 256, 32 and
// 4 fp64 sums over 16384 counts). Every sum is of fp32 counts in fp64 and is
// exact, so its value does not depend on the order of the additions, and the
// donors are those of the one-by-one definition bit for bit.
// The settle loop is one wave's dependent chain (fp64 multiply, compares,
// ballot, lane reads, fp64 updates), a few hundred cycles per draw; about a
// third of the candidates are right at the first SIFT-like check, and a miss
// costs one 16-cluster walk step (an LDS read and a 16-lane fp64 scan).
constexpr int kSpecK = 16384;
// Draws speculated per round (lanes 0 .. kSpecRound - 1 of wave 0). Rounds of
// 8, 16, 32 and 64 draws cost within 4% of each other over whole runs (the
// fresher candidates of short rounds hit more often, but each round starts
// with its own tree search); 32 was the fastest.
constexpr int kSpecRound = 32;

// First of N consecutive sums whose running total from acc exceeds t (N if
// none); acc becomes the running total before it.
template <int N>
__device__ __forceinline__ int pick_child(const double* s, double t, double& acc) {
  double v[N];
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    const double2 p = *reinterpret_cast<const double2*>(s + i);
    v[i] = p.x;
    v[i + 1] = p.y;
  }
  double run[N];
  run[0] = acc + v[0];
#pragma unroll
  for (int i = 1; i < N; ++i) run[i] = run[i - 1] + v[i];
  int r = N;
  double before = acc;
#pragma unroll
  for (int i = N - 1; i >= 0; --i)
    if (run[i] > t) {
      r = i;
      before = i > 0 ? run[i - 1] : acc;
    }
  acc = before;
  return r;
}

// Inclusive fp64 scan within each row of 16 lanes.
__device__ __forceinline__ double row_scan16_f64(double v) {
  v += dpp_move_f64<0x111, 0xF>(v);  // row_shr:1
  v += dpp_move_f64<0x112, 0xF>(v);  // row_shr:2
  v += dpp_move_f64<0x114, 0xF>(v);  // row_shr:4
  v += dpp_move_f64<0x118, 0xF>(v);  // row_shr:8
  return v;
}

__global__ __launch_bounds__(1024) void revive_spec_kernel(ReviveArgs A) {
  constexpr int RR = kSpecRound;
  constexpr int RV = kSpecK / 1024;  // clusters per thread in the set-up
  __shared__ double dtmp[16];
  __shared__ int itmp[16];
  __shared__ __attribute__((aligned(16))) float wc[kSpecK + 64];  // live counts, compacted
  __shared__ int lidx[kSpecK];                                      // their clusters
  __shared__ __attribute__((aligned(16))) double t1[kSpecK / 8];  // sums of 8 counts
  __shared__ __attribute__((aligned(16))) double t2[kSpecK / 64];
  __shared__ __attribute__((aligned(16))) double t3[kSpecK / 512];
  __shared__ __attribute__((aligned(16))) double t4[kSpecK / 4096];
  __shared__ float sink[64];  // target of the stores of lanes that do not write
  __shared__ int s_ndead;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int k = A.k;
  if (tid == 0) A.nheads[0] = 0;

  // ---- threshold, dead list, compacted live counts ---------------------------
  // thread tid owns clusters RV tid .. RV tid + RV - 1, read once
  float nv[RV];
#pragma unroll
  for (int e = 0; e < RV; ++e) {
    const int j = RV * tid + e;
    nv[e] = j < k ? A.N[j] : 0.0f;
  }
  double loc = 0.0;
#pragma unroll
  for (int e = 0; e < RV; ++e) loc += (double)nv[e];
  const double total = block_sum<double, 1024>(loc, dtmp);
  const double th = A.empty_only ? 0.5 : A.thr * (total / (double)k);
  unsigned deadm = 0;
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < RV; ++e) {
    const int j = RV * tid + e;
    if (j < k) {
      const int dd = ((double)nv[e] < th) ? 1 : 0;
      A.flags[j] = dd;
      A.n0[j] = nv[e];
      deadm |= (unsigned)dd << e;
      cnt += dd;
    }
  }
  const int incl = block_incl_scan<int, 1024>(cnt, itmp);
  if (tid == 1023) s_ndead = incl;
  int wpos = incl - cnt;                   // dead clusters before this thread's
  int lpos = min(k, RV * tid) - wpos;      // live clusters before this thread's
#pragma unroll
  for (int e = 0; e < RV; ++e) {
    const int j = RV * tid + e;
    if (j < k) {
      if ((deadm >> e) & 1u) {
        A.dead[wpos++] = j;
      } else {
        wc[lpos] = nv[e];
        lidx[lpos] = j;
        ++lpos;
      }
    }
  }
  __threadfence_block();
  __syncthreads();
  const int ndead = s_ndead;
  const int M = k - ndead;  // live clusters
  if (A.count_only) {
    if (tid == 0) A.counters[2] = ndead;
    return;
  }
  if (ndead == 0 || M == 0) return;  // nothing to revive, or no donor exists
  for (int q = tid; q < ndead; q += 1024)
    A.udraw[q] = revive_uniform(A.seed, A.step, (uint64_t)A.dead[q]);
  for (int m = M + tid; m < kSpecK + 64; m += 1024) wc[m] = 0.0f;
  __threadfence_block();
  __syncthreads();
  for (int i = tid; i < kSpecK / 8; i += 1024) {
    const float4 a = *reinterpret_cast<const float4*>(&wc[8 * i]);
    const float4 b = *reinterpret_cast<const float4*>(&wc[8 * i + 4]);
    t1[i] = (((double)a.x + (double)a.y) + ((double)a.z + (double)a.w)) +
            (((double)b.x + (double)b.y) + ((double)b.z + (double)b.w));
  }
  __syncthreads();
  auto sum8 = [](const double* s) {
    return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
  };
  for (int i = tid; i < kSpecK / 64; i += 1024) t2[i] = sum8(&t1[8 * i]);
  __syncthreads();
  if (tid < kSpecK / 512) t3[tid] = sum8(&t2[8 * tid]);
  __syncthreads();
  if (tid < kSpecK / 4096) t4[tid] = sum8(&t3[8 * tid]);
  __syncthreads();

  // ---- draws (wave 0) ---------------------------------------------------------
  if (wave == 0) {
    double T = (t4[0] + t4[1]) + (t4[2] + t4[3]);  // live total
    int64_t logc = A.counters[1];
    // the first round's dead clusters and draws; later rounds load theirs one
    // round ahead
    int dl = lane < ndead ? A.dead[lane] : 0;
    double u = lane < ndead ? A.udraw[lane] : 0.0;
    for (int d0 = 0; d0 < ndead; d0 += RR) {
      const int nb = min(RR, ndead - d0);
      const bool act = lane < nb;
      const int dn = d0 + RR + lane;
      const int dl_next = dn < ndead ? A.dead[dn] : 0;
      const double u_next = dn < ndead ? A.udraw[dn] : 0.0;
      // 1. candidate from the round-start sums; a target at or past the total
      // (no cluster exceeds it) takes position M, with L = H = T
      const double t0 = u * T;
      double acc = 0.0;
      int m = M;
      double L = T, H = T;
      const int i4 = pick_child<4>(t4, t0, acc);
      if (i4 < 4) {
        const int n3 = 8 * i4 + min(pick_child<8>(&t3[8 * i4], t0, acc), 7);
        const int n2 = 8 * n3 + min(pick_child<8>(&t2[8 * n3], t0, acc), 7);
        const int n1 = 8 * n2 + min(pick_child<8>(&t1[8 * n2], t0, acc), 7);
        double w8[8];
        const float4 a = *reinterpret_cast<const float4*>(&wc[8 * n1]);
        const float4 b = *reinterpret_cast<const float4*>(&wc[8 * n1 + 4]);
        w8[0] = a.x; w8[1] = a.y; w8[2] = a.z; w8[3] = a.w;
        w8[4] = b.x; w8[5] = b.y; w8[6] = b.z; w8[7] = b.w;
        const int i0 = min(pick_child<8>(w8, t0, acc), 7);
        m = 8 * n1 + i0;
        L = acc;
        H = acc + w8[i0];
      }
      // half the candidate's current count (0 at position M), as the split
      // would take it, in fp32 and fp64; the current counts of its two
      // neighbours on each side (0 before position 0 and past M)
      float half = wc[m] * 0.5f;
      double halfd = (double)half;
      float wl1 = m >= 1 ? wc[max(m - 1, 0)] : 0.0f, wl2 = m >= 2 ? wc[max(m - 2, 0)] : 0.0f;
      float wr1 = wc[m + 1], wr2 = wc[m + 2];  // m + 2 <= M + 2: zero padding
      // waited for here, so that the loop below never waits for its own stores
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      double Tq = T;
      int rec_m = 0;
      float rec_n = 0.0f;
      // 2. settle the draws in order
      for (int q = 0; q < nb; ++q) {
        const double t = u * Tq;
        // two ballots and a scalar AND: a ballot of the combined predicate
        // goes through a vector select and compare on the draw's chain
        const uint64_t okm = __ballot(L <= t) & __ballot(t < H);
        int ms;
        float nh;
        double nhd;
        if ((okm >> q) & 1ull) {
          ms = __builtin_amdgcn_readlane(m, q);
          nh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(half), q));
          nhd = readlane_f64(halfd, q);
        } else {
          const uint64_t rightm = __ballot(t >= H);
          const double tq = readlane_f64(t, q);
          const int mq = __builtin_amdgcn_readlane(m, q);
          ms = -1;
          float cn = 0.0f;
          if ((rightm >> q) & 1ull) {
            // right of the candidate: cum(p0 - 1) = c <= tq; first its two
            // neighbours (a count of 0 is padding past M and never taken)
            double c = readlane_f64(H, q);
            const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wr1), q));
            const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wr2), q));
            const double c1 = c + (double)r1, c2 = c1 + (double)r2;
            int p0 = mq + 3;
            if (tq < c1) {
              ms = mq + 1;
              cn = r1;
              p0 = M;  // found
            } else if (tq < c2) {
              ms = mq + 2;
              cn = r2;
              p0 = M;
            }
            c = c2;
            for (; p0 < M; p0 += 16) {
              const float w = wc[p0 + (lane & 15)];  // zero past M
              const double v = row_scan16_f64((double)w);
              const uint64_t hm = __ballot(c + v > tq) & 0xFFFFull;
              if (hm) {
                const int i = __ffsll((unsigned long long)hm) - 1;
                ms = p0 + i;
                cn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), i));
                break;
              }
              c += readlane_f64(v, 15);
            }
            if (ms < 0) {  // the target reaches the total: the last live cluster
              ms = M - 1;
              cn = wc[M - 1];
            }
          } else {
            // left of the candidate: cum(p0) = c > tq; first its two neighbours
            double c = readlane_f64(L, q);
            const float l1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl1), q));
            const float l2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl2), q));
            const double c1 = c - (double)l1, c2 = c1 - (double)l2;
            int p0 = mq - 3;
            if (c1 <= tq) {
              ms = mq - 1;
              cn = l1;
              p0 = -1;  // found
            } else if (c2 <= tq) {
              ms = mq - 2;
              cn = l2;
              p0 = -1;
            }
            c = c2;
            for (; p0 >= 0; p0 -= 16) {
              const int pos = p0 - (lane & 15);
              const float w = pos >= 0 ? wc[max(pos, 0)] : 0.0f;
              const double v = row_scan16_f64((double)w);
              const uint64_t hm = __ballot(pos >= 0) & __ballot(c - v <= tq) & 0xFFFFull;
              if (hm) {
                const int i = __ffsll((unsigned long long)hm) - 1;
                ms = p0 - i;
                cn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), i));
                break;
              }
              c -= readlane_f64(v, 15);
            }
            if (ms < 0) {  // not reachable with exact sums: cum(-1) = 0 <= tq
              ms = 0;
              cn = wc[0];
            }
          }
          __builtin_amdgcn_s_waitcnt(0xC07F);  // its LDS reads are done before the join
          nh = cn * 0.5f;
          nhd = (double)nh;
        }
        // the donor's count halves (lane 0 stores it; the others store to the sink)
        *(lane == 0 ? &wc[ms] : &sink[lane]) = nh;
        Tq -= nhd;
        H -= ms <= m ? nhd : 0.0;
        L -= ms < m ? nhd : 0.0;
        const bool hit = ms == m;
        const float hh = half * 0.5f;
        half = hit ? hh : half;
        halfd = hit ? (double)hh : halfd;
        const int dm = ms - m;  // the neighbours' counts halve too
        wl2 = dm == -2 ? nh : wl2;
        wl1 = dm == -1 ? nh : wl1;
        wr1 = dm == 1 ? nh : wr1;
        wr2 = dm == 2 ? nh : wr2;
        rec_m = lane == q ? ms : rec_m;
        rec_n = lane == q ? nh : rec_n;
      }
      // 3. the tree learns the round's halvings; outputs of the round
      if (act) {
        const double nd = (double)rec_n;
        atomicAdd(&t1[rec_m >> 3], -nd);
        atomicAdd(&t2[rec_m >> 6], -nd);
        atomicAdd(&t3[rec_m >> 9], -nd);
        atomicAdd(&t4[rec_m >> 12], -nd);
        const int ci = lidx[rec_m];
        A.N[dl] = rec_n;
        A.pair_i[d0 + lane] = ci;
        A.pair_n[d0 + lane] = rec_n;
        if (A.log && logc + lane < A.log_cap) {
          A.log[3 * (logc + lane)] = (int32_t)A.step;
          A.log[3 * (logc + lane) + 1] = dl;
          A.log[3 * (logc + lane) + 2] = ci;
        }
      }
      if (A.log) logc = min(A.log_cap, logc + nb);
      T = Tq;
      dl = dl_next;
      u = u_next;
    }
    if (lane == 0) A.counters[1] = logc;
  }
  __syncthreads();
  // the donors' halved counts (dead clusters were written by the rounds)
  for (int m = tid; m < M; m += 1024) A.N[lidx[m]] = wc[m];
  __threadfence_block();
  __syncthreads();
  revive_chains(A, ndead, itmp);
}

// One wave per donor chain: apply its splits of the running sums in order.
__global__ __launch_bounds__(256) void split_kernel(ReviveArgs A) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= A.nheads[0]) return;
  const int d = A.d;
  const int qh = A.heads[w];
  const int base = A.cbase[qh], len = A.clen[qh];
  for (int r = 0; r < len; ++r) {
    const int q = A.list[base + r];
    const int i = A.pair_i[q];
    const int j = A.dead[q];
    const float Nh = A.pair_n[q];
    if (A.N2 && lane == 0) {  // the counts are final once revive_kernel has run
      A.N2[j] = A.N[j];
      A.N2[i] = A.N[i];
    }
    float ni = 0.0f, nj = 0.0f;
    int qni = 0, qnj = 0;  // |q|^2 of the int8 codes, exact
    U64x4 wd = {0, 0, 0, 0};
    for (int e = lane, it = 0; e < d; e += 64, ++it) {
      if ((it & 3) == 0)
        wd = philox((uint64_t)j, A.step, (uint64_t)(e >> 8), kStreamSign, A.seed, 0);
      const uint64_t word = (it & 3) == 0 ? wd.w0 : (it & 3) == 1 ? wd.w1 : (it & 3) == 2 ? wd.w2 : wd.w3;
      const float sg = ((word >> (e & 63)) & 1) ? -1.0f : 1.0f;
      const size_t ii = (size_t)i * d + e, jj = (size_t)j * d + e;
      const float half = A.S[ii] * 0.5f;
      const float sj = __fmul_rn(half, 1.0f + kSplitEps * sg);
      const float si = __fmul_rn(half, 1.0f - kSplitEps * sg);
      A.S[jj] = sj;
      A.S[ii] = si;
      if (A.S2) {  // the slow pair of both halves restarts from the split values
        A.S2[jj] = sj;
        A.S2[ii] = si;
      }
      float cj = __fdiv_rn(sj, Nh), ci = __fdiv_rn(si, Nh);
      A.C[jj] = cj;
      A.C[ii] = ci;
      if (A.Chat) {
        const bool hf = A.chat_f16;
        const uint16_t hj = to_half_rne(conv_in(cj, A.sshift, A.sscale, e), hf),
                       hi = to_half_rne(conv_in(ci, A.sshift, A.sscale, e), hf);
        A.Chat[jj] = hj;
        A.Chat[ii] = hi;
        cj = half_to_f32(hj, hf);
        ci = half_to_f32(hi, hf);
      } else if (A.Cf) {
        const uint32_t fj = f32_to_e4m3(conv_in(cj, A.sshift, A.sscale, e)),
                       fi = f32_to_e4m3(conv_in(ci, A.sshift, A.sscale, e));
        A.Cf[jj] = (uint8_t)fj;
        A.Cf[ii] = (uint8_t)fi;
        cj = e4m3_to_f32(fj);
        ci = e4m3_to_f32(fi);
      } else if (A.Cq) {
        const int8_t qj = to_code(cj, A.cq_u8), qi = to_code(ci, A.cq_u8);
        A.Cq[jj] = qj;
        A.Cq[ii] = qi;
        qni += (int)qi * (int)qi;
        qnj += (int)qj * (int)qj;
        continue;
      }
      ni += ci * ci;
      nj += cj * cj;
    }
    if (A.sph) {
      // spherical e-means: both halves rescaled to norm 1, then rounded to Chat
      wave_normalize(A.C + (size_t)i * d, d, lane);
      wave_normalize(A.C + (size_t)j * d, d, lane);
      if (A.Chat)
        for (int e = lane; e < d; e += 64) {
          A.Chat[(size_t)i * d + e] = to_half_rne(A.C[(size_t)i * d + e], A.chat_f16);
          A.Chat[(size_t)j * d + e] = to_half_rne(A.C[(size_t)j * d + e], A.chat_f16);
        }
      if (lane == 0) {
        A.bias[i] = 0.0f;
        A.bias[j] = 0.0f;
      }
      continue;
    }
    if (A.Cq) {
      qni = wave_sum(qni);
      qnj = wave_sum(qnj);
      if (lane == 0) {
        reinterpret_cast<int32_t*>(A.bias)[i] = -qni;
        reinterpret_cast<int32_t*>(A.bias)[j] = -qnj;
      }
      continue;
    }
    ni = wave_sum(ni);
    nj = wave_sum(nj);
    if (lane == 0) {
      A.bias[i] = -0.5f * ni;
      A.bias[j] = -0.5f * nj;
    }
  }
}

__global__ __launch_bounds__(1024) void pass_stats_kernel(int32_t* pass_counts, int k,
                                                          double* sums, int reset) {
  __shared__ double tmp[16];
  double s2 = 0.0, s1 = 0.0;
  for (int j = threadIdx.x; j < k; j += 1024) {
    const double n = (double)pass_counts[j];
    s2 += n * n;
    s1 += n;
    if (reset) pass_counts[j] = 0;
  }
  s2 = block_sum<double, 1024>(s2, tmp);
  s1 = block_sum<double, 1024>(s1, tmp);
  if (threadIdx.x == 0) {
    sums[0] += s2;
    sums[1] += s1;
  }
}

__global__ void finalize_kernel(int k, int d, const int32_t* pass_counts, const float* LS,
                                float* C) {
  const size_t total = (size_t)k * d;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int j = (int)(idx / d);
    const int n = pass_counts[j];
    if (n > 0) C[idx] = __fdiv_rn(LS[idx], (float)n);
  }
}

// Spherical e-means: rows of C rescaled to norm 1 in place, one wave per row.
__global__ __launch_bounds__(256) void normalize_rows_kernel(float* C, int k, int d) {
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j < k) wave_normalize(C + (size_t)j * d, d, threadIdx.x & 63);
}

// Spherical closing step: one wave per cluster, the exact mean of the last
// pass rescaled to norm 1.
__global__ __launch_bounds__(256) void finalize_sph_kernel(int k, int d,
                                                           const int32_t* pass_counts,
                                                           const float* LS, float* C) {
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= k) return;
  const int n = pass_counts[j];
  if (n <= 0) return;
  const size_t base = (size_t)j * d;
  for (int e = lane; e < d; e += 64) C[base + e] = __fdiv_rn(LS[base + e], (float)n);
  wave_normalize(C + base, d, lane);
}

}  // namespace

hipError_t launch_sample_rows(const PermKey& pk, uint64_t start, int count, uint32_t* rows,
                              hipStream_t st) {
  if (count <= 0) return hipSuccess;
  // several slots per thread only once the batch keeps 2^18 threads busy
  int q = count >> 18;
  q = q < 1 ? 1 : (q > 8 ? 8 : q);
  const int threads = (count + q - 1) / q;
  sample_rows_kernel<<<(threads + 255) / 256, 256, 0, st>>>(pk, start, count, q, rows);
  return hipGetLastError();
}

hipError_t launch_convert_rows(const float* X, int d, const uint32_t* rows, int nrows, int fmt,
                               const float* shift, float scale, void* out, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  auto* o = static_cast<unsigned char*>(out);
  const bool vec = d % 8 == 0 && (uintptr_t)X % 16 == 0 && (uintptr_t)o % 16 == 0 &&
                   (uintptr_t)shift % 16 == 0;
  const int64_t work = (int64_t)nrows * (vec ? d / 8 : d);
  const unsigned grid = (unsigned)((work + 255) / 256);
#define EMK_CONV(F)                                                                              \
  do {                                                                                           \
    if (vec)                                                                                     \
      convert_rows_kernel<F, true><<<grid, 256, 0, st>>>(X, d, rows, nrows, shift, scale, o);   \
    else                                                                                         \
      convert_rows_kernel<F, false><<<grid, 256, 0, st>>>(X, d, rows, nrows, shift, scale, o);  \
  } while (0)
  if (fmt == 3)
    EMK_CONV(3);
  else if (fmt == 4)
    EMK_CONV(4);
  else
    EMK_CONV(1);
#undef EMK_CONV
  return hipGetLastError();
}

hipError_t launch_sample_rows_i32(const PermKey& pk, uint64_t start, int count, int32_t* rows,
                                  hipStream_t st) {
  if (count <= 0) return hipSuccess;
  sample_rows_i32_kernel<<<(count + 255) / 256, 256, 0, st>>>(pk, start, count, rows);
  return hipGetLastError();
}

hipError_t launch_init_centroids(int dt, const void* X, int d, const PermKey& pk, int k,
                                 float* C, bool sph, hipStream_t st) {
  init_centroids_kernel<<<(k + 3) / 4, 256, 0, st>>>(static_cast<const unsigned char*>(X), dt, d,
                                                     pk, k, C, sph ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_prep(const float* C, int k, int d, float* bias, uint16_t* Chat, bool chat_f16,
                       int8_t* Cq, bool cq_u8, uint8_t* Cf, const float* sshift, float sscale,
                       bool sph, hipStream_t st) {
  prep_kernel<<<(k + 3) / 4, 256, 0, st>>>(C, k, d, bias, Chat, chat_f16 ? 1 : 0, Cq,
                                           cq_u8 ? 1 : 0, Cf, sshift, sscale, sph ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_scan(int32_t* counts, int k, int R, int32_t* off, int32_t* cursor,
                       int2* ovf, int32_t* ovf_n, int32_t* acc, hipStream_t st) {
  // items of R rows, R a power of two: the kernel divides by shifting
  if (R <= 0 || (R & (R - 1)) != 0) return hipErrorInvalidValue;
  const int rsh = __builtin_ctz((unsigned)R);
  scan_kernel<<<1, 1024, 0, st>>>(counts, k, R, rsh, off, cursor, ovf, ovf_n, acc);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* labels, const uint32_t* rows, int nb, int k,
                          int32_t* cursor, uint32_t* order, int2* olab, int32_t* out_labels,
                          hipStream_t st) {
  if (nb <= 0) return hipSuccess;
  scatter_kernel<<<(nb + 255) / 256, 256, 0, st>>>(labels, rows, nb, k, cursor, order, olab,
                                                   out_labels);
  return hipGetLastError();
}

hipError_t launch_label_hist(const int32_t* labels, int nb, int k, int32_t* counts,
                             int32_t* bad, hipStream_t st) {
  if (nb <= 0) return hipSuccess;
  label_hist_kernel<<<(nb + 255) / 256, 256, 0, st>>>(labels, nb, k, counts, bad);
  return hipGetLastError();
}

hipError_t launch_closing_add(int k, int d, int32_t* counts, float* s_acc, int32_t* pass_counts,
                              float* LS, hipStream_t st) {
  closing_add_kernel<<<(k + 3) / 4, 256, 0, st>>>(k, d, counts, s_acc, pass_counts, LS);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_group_dt(const unsigned char* x, int d, bool vec, int ncol,
                                  const uint32_t* order, const int2* olab, const int32_t* off,
                                  const int2* ovf, const int32_t* ovf_n, int k, int R,
                                  long long items, float* s_acc, int add, int nb,
                                  hipStream_t st) {
  // narrow rows: spans of consecutive clusters, one lane per 4-, 8- or 16-byte unit
  constexpr int ES = DT == 0 ? 4 : (DT == 1 || DT == 4) ? 2 : 1;
  const size_t rowbytes = (size_t)d * ES;
  int ub = 0;
  for (int cand = 4; cand <= 16; cand *= 2)  // at most 4 elements per lane per row
    if (!ub && cand / ES <= 4 && rowbytes % cand == 0 && rowbytes / cand <= 64 &&
        (uintptr_t)x % cand == 0)
      ub = cand;
  if (ub && olab && (long long)nb <= 8LL * k) {
    // at most 8 rows per cluster on average: windows of 8 slots, one wave each
    const dim3 grid((unsigned)((((long long)nb + 7) / 8 + 3) / 4)), block(256);
    if (ub == 4)
      group_win_kernel<DT, 4, 8, 8><<<grid, block, 0, st>>>(x, d, olab, off, k, nb, s_acc, add);
    if constexpr (ES >= 2)
      if (ub == 8)
        group_win_kernel<DT, 8, 8, 8><<<grid, block, 0, st>>>(x, d, olab, off, k, nb, s_acc, add);
    if constexpr (ES >= 4)
      if (ub == 16)
        group_win_kernel<DT, 16, 8, 8><<<grid, block, 0, st>>>(x, d, olab, off, k, nb, s_acc,
                                                                add);
    return hipGetLastError();
  }
  if (ub) {
    // about 16 rows per span: C clusters of nb / k rows on average
    const double avg = (double)nb / (double)k;
    int C = (int)(16.0 / (avg > 1.0 ? avg : 1.0));
    C = C < 1 ? 1 : (C > 32 ? 32 : C);
    const int nA = (k + C - 1) / C;
    const long long waves = (long long)nA + nb / R;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (ub == 4 && C == 1)  // clusters of 16 rows or more on average
      group_span_kernel<DT, 4, 32><<<grid, block, 0, st>>>(x, d, order, off, ovf, ovf_n, k, R, C,
                                                            nA, s_acc, add);
    else if (ub == 4)
      group_span_kernel<DT, 4><<<grid, block, 0, st>>>(x, d, order, off, ovf, ovf_n, k, R, C, nA,
                                                        s_acc, add);
    if constexpr (ES >= 2)
      if (ub == 8)
        group_span_kernel<DT, 8><<<grid, block, 0, st>>>(x, d, order, off, ovf, ovf_n, k, R, C,
                                                          nA, s_acc, add);
    if constexpr (ES >= 4)
      if (ub == 16)
        group_span_kernel<DT, 16><<<grid, block, 0, st>>>(x, d, order, off, ovf, ovf_n, k, R, C,
                                                           nA, s_acc, add);
    return hipGetLastError();
  }
  if (ncol <= 64) {
    const dim3 wgrid((unsigned)((items + 3) / 4)), wblock(256);
    if (vec)
      group_wave_kernel<DT, true>
          <<<wgrid, wblock, 0, st>>>(x, d, order, off, ovf, ovf_n, k, R, s_acc, add);
    else
      group_wave_kernel<DT, false>
          <<<wgrid, wblock, 0, st>>>(x, d, order, off, ovf, ovf_n, k, R, s_acc, add);
    return hipGetLastError();
  }
  int nt = 256;
  if (ncol < 256) nt = (((256 / ncol) * ncol + 63) / 64) * 64;
  const dim3 grid((unsigned)items), block(nt);
  if (vec)
    group_kernel<DT, true><<<grid, block, 0, st>>>(x, d, order, off, ovf, ovf_n, k, R, s_acc, add);
  else
    group_kernel<DT, false><<<grid, block, 0, st>>>(x, d, order, off, ovf, ovf_n, k, R, s_acc, add);
  return hipGetLastError();
}

int group_rows(int dt, int d) {
  const int es = dt == 0 ? 4 : (dt == 1 || dt == 4) ? 2 : 1;
  // narrow rows (one wave per item) take longer items, so that clusters of a
  // few hundred rows are summed by one wave without atomics (4.8 instead of
  // 3.3 TB/s on 4M-row bf16 batches of 64-row clusters); wide rows (one
  // workgroup per item) keep 64, which spreads the large clusters of skewed
  // data over more workgroups
  return (int64_t)d * es <= 1024 ? kNarrowRows : 64;
}

hipError_t launch_group(int dt, const void* X, int d, const uint32_t* order,
                        const int2* olab, const int32_t* off, const int2* ovf,
                        const int32_t* ovf_n, int k, int R, int nb, float* s_acc, bool add,
                        hipStream_t st) {
  if (nb <= 0) return hipSuccess;
  // work items: one per cluster plus at most nb / R overflow items
  const long long items = (long long)k + nb / R;
  const auto* x = static_cast<const unsigned char*>(X);
  // a vector unit is 16 B (4 fp32, 8 bf16 / fp16) or, for int8 / E4M3 codes, 4 B
  const bool codes = dt == 2 || dt == 3 || dt == 5;
  const int per = (dt == 1 || dt == 4) ? 8 : 4;
  const bool aligned = (uintptr_t)X % (codes ? 4 : 16) == 0;
  const bool vec = aligned && d % per == 0;
  const int ncol = vec ? d / per : d;
  const int a = add ? 1 : 0;
  if (dt == 1)
    return launch_group_dt<1>(x, d, vec, ncol, order, olab, off, ovf, ovf_n, k, R, items, s_acc, a,
                              nb, st);
  if (dt == 2)
    return launch_group_dt<2>(x, d, vec, ncol, order, olab, off, ovf, ovf_n, k, R, items, s_acc, a,
                              nb, st);
  if (dt == 3)
    return launch_group_dt<3>(x, d, vec, ncol, order, olab, off, ovf, ovf_n, k, R, items, s_acc, a,
                              nb, st);
  if (dt == 4)
    return launch_group_dt<4>(x, d, vec, ncol, order, olab, off, ovf, ovf_n, k, R, items, s_acc, a,
                              nb, st);
  if (dt == 5)
    return launch_group_dt<5>(x, d, vec, ncol, order, olab, off, ovf, ovf_n, k, R, items, s_acc, a,
                              nb, st);
  return launch_group_dt<0>(x, d, vec, ncol, order, olab, off, ovf, ovf_n, k, R, items, s_acc, a,
                              nb, st);
}

hipError_t launch_ema(int k, int d, float a, float b, int32_t* counts, float* s_acc, float* N,
                      float* S, float* C, float* bias, uint16_t* Chat, bool chat_f16, int8_t* Cq,
                      bool cq_u8, uint8_t* Cf, int32_t* pass_counts, float* LS, bool sph,
                      float beta, float b2, float* N2, float* S2, const float* sshift,
                      float sscale, hipStream_t st) {
  const dim3 grid((k + 3) / 4), block(256);
  const int sp = sph ? 1 : 0;
#define EMK_EMA(SF)                                                                        \
  ema_kernel<SF><<<grid, block, 0, st>>>(k, d, a, b, counts, s_acc, N, S, C, bias, Chat, Cq, \
                                         Cf, pass_counts, LS, sp, beta, b2, N2, S2, sshift, sscale)
  if (Chat && chat_f16)
    EMK_EMA(4);
  else if (Chat)
    EMK_EMA(1);
  else if (Cq && cq_u8)
    EMK_EMA(5);
  else if (Cq)
    EMK_EMA(2);
  else if (Cf)
    EMK_EMA(3);
  else
    EMK_EMA(0);
#undef EMK_EMA
  return hipGetLastError();
}

__global__ void scale_kernel(float* a, int64_t n, float f) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) a[i] *= f;
}

hipError_t launch_scale(float* a, int64_t n, float f, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  scale_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(a, n, f);
  return hipGetLastError();
}

hipError_t launch_slow_final(int k, int d, const float* N2, const float* S2, const float* C,
                             float* out, bool sph, hipStream_t st) {
  slow_final_kernel<<<(k + 3) / 4, 256, 0, st>>>(k, d, N2, S2, C, out, sph ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_revive(const ReviveArgs& a, hipStream_t st) {
  const int v = (a.k + 4095) / 4096;
  if (a.k <= kSpecK)
    revive_spec_kernel<<<1, 1024, 0, st>>>(a);
  else if (v <= 1)
    revive_kernel<1><<<1, 1024, 0, st>>>(a);
  else if (v <= 2)
    revive_kernel<2><<<1, 1024, 0, st>>>(a);
  else if (v <= 4)
    revive_kernel<4><<<1, 1024, 0, st>>>(a);
  else if (v <= 8)
    revive_kernel<8><<<1, 1024, 0, st>>>(a);
  else if (v <= 16)
    revive_kernel<16><<<1, 1024, 0, st>>>(a);
  else
    revive_kernel<0><<<1, 1024, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.count_only) return e;
  split_kernel<<<(a.k + 3) / 4, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_pass_stats(int32_t* pass_counts, int k, double* sums, int reset,
                             hipStream_t st) {
  pass_stats_kernel<<<1, 1024, 0, st>>>(pass_counts, k, sums, reset);
  return hipGetLastError();
}

hipError_t launch_normalize_rows(float* C, int k, int d, hipStream_t st) {
  normalize_rows_kernel<<<(k + 3) / 4, 256, 0, st>>>(C, k, d);
  return hipGetLastError();
}

hipError_t launch_finalize(int k, int d, const int32_t* pass_counts, const float* LS, float* C,
                           bool sph, hipStream_t st) {
  if (sph) {
    finalize_sph_kernel<<<(k + 3) / 4, 256, 0, st>>>(k, d, pass_counts, LS, C);
    return hipGetLastError();
  }
  const size_t total = (size_t)k * d;
  const size_t want = (total + 255) / 256;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  finalize_kernel<<<blocks, 256, 0, st>>>(k, d, pass_counts, LS, C);
  return hipGetLastError();
}

}  // namespace emk
