// Nearest-centroid assignment for int8 codes and uint8 data of small
// dimension (d = 32 * KS, d <= 256) on gfx950: points resident in registers,
// centroids streamed, exact integer scores.
//
// A wave keeps its points as MFMA B operands in registers for the whole sweep
// over the centroids (d bytes per point: 128 points at d <= 128, 96 up to
// d = 192, 64 above), and the only streamed data are the centroid code
// panels, shared by the eight waves of the workgroup through LDS. The eight
// waves form 8 / CG point groups of CG waves; the CG waves of a group hold
// the same points and take every CG-th 32-centroid block of a panel, so a
// small batch still spreads over all compute units (CG = 1 for large
// batches: the least panel traffic). v_mfma_i32_32x32x32_i8 tiles put 32
// centroids on M and 32 points on N; each lane holds 16 consecutive bytes of
// a row per k-step (lane / 32 picks the half of the 32-byte k-step). After
// the KS k-steps each lane holds 16 exact dot products x.q of one point.
//
// The score is the integer 2 x.q - |q|^2 (bias = -|q|^2 as int32), kept, as
// the float kernels do, at its maximum with the lowest index on ties. The fold
// needs no branch: the panel store turns each bias into the key
// 16 bias + 15 - slot (slot = the row's place among a lane's 16 accumulator
// values), so 32 x.q + key is 16 score + 15 - slot, a value whose maximum over
// the block is the block's best score with its lowest slot. |score| < 2^24 for
// d <= 256 (|x.q| <= 2^22, |q|^2 <= 2^22), so the packed value stays inside
// int32, and rows past k get a key of -2^30, below every real packed value.
// A block replaces the lane's best only with a higher score (not a tie), so
// earlier blocks keep ties and the lane ends with its lowest-index maximum.
//
// uint8 rows are shifted by -128 into int8 (u ^ 0x80 read as int8 is u - 128)
// once, as the points are loaded; the centroid codes are stored shifted the
// same way, so every distance is unchanged. With d <= 43919 no score leaves
// int32 (the int8 search's bound), far above the d <= 256 of this kernel.
#include <atomic>

#include "kernels.hpp"

namespace emk {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;               // two waves per SIMD: one folds while the other multiplies
constexpr int kThreads = 64 * kWaves;
constexpr int kTC = 256;                // centroids per LDS panel
constexpr int kMasked = -(1 << 30);     // key of a row past k

// 32-point blocks a wave holds: as many as the registers allow.
constexpr __host__ __device__ int pblocks(int ks) { return ks <= 4 ? 4 : ks <= 6 ? 3 : 2; }

__device__ __forceinline__ int max3i(int a, int b, int c) { return max(max(a, b), c); }

template <int KS, bool U8, int CG>
__global__ __launch_bounds__(kThreads, 1) void assign_i8r_kernel(
    const uint8_t* __restrict__ X, const uint32_t* __restrict__ rows, int nrows,
    const int8_t* __restrict__ Cq, const int32_t* __restrict__ bias, int k,
    int32_t* __restrict__ labels, float* __restrict__ dists, int32_t* __restrict__ counts,
    double* __restrict__ obj) {
  constexpr int d = 32 * KS;
  constexpr int kPB = pblocks(KS);           // 32-point blocks per wave
  constexpr int kTPw = 32 * kPB;             // points per wave (and per point group)
  constexpr int kTP = kTPw * (kWaves / CG);  // points per workgroup
  constexpr int kStride = d + 16;            // 16 consecutive rows hit 16 disjoint 4-bank groups
  constexpr int CPR = d / 16;                // 16-byte chunks per centroid row
  constexpr int PER = kTC * CPR / kThreads;  // chunk loads per thread per panel
  static_assert(kTC * CPR % kThreads == 0, "whole chunk loads per thread");
  __shared__ __attribute__((aligned(16))) unsigned char lc[2][kTC * kStride];
  __shared__ __attribute__((aligned(16))) int32_t lb[2][kTC];
  __shared__ int32_t m_s[CG][kTP];
  __shared__ int m_j[CG][kTP];
  __shared__ int32_t m_x[kTP];
  __shared__ double red[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;  // which 16 bytes of each 32-byte k-step this lane holds
  const int pg = wave / CG;    // point group
  const int cg = wave % CG;    // first 32-centroid block of each panel this wave takes
  const int tile0 = blockIdx.x * kTP;

  // ---- points of this wave into registers (B operands) ----------------------
  u32x4 pB[kPB][KS];
  int xn[kPB];
#pragma unroll
  for (int pb = 0; pb < kPB; ++pb) {
    const int slot = min(tile0 + pg * kTPw + pb * 32 + (lane & 31), nrows - 1);
    const size_t r = rows ? (size_t)rows[slot] : (size_t)slot;
    const unsigned char* row = X + r * d;
    int s = 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = *reinterpret_cast<const u32x4*>(row + 32 * ks + 16 * half);
      if constexpr (U8) w ^= 0x80808080u;
      pB[pb][ks] = w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int v = (int)(int8_t)(w[e] >> (8 * b));
          s += v * v;
        }
    }
    xn[pb] = s + __shfl_xor(s, 32, 64);
  }

  // ---- centroid panel staging ------------------------------------------------
  const int npan = (k + kTC - 1) / kTC;
  u32x4 rc[PER];
  int32_t rkey = 0;
  auto gload = [&](int panel) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + kThreads * i;  // chunk id: row q / CPR, chunk q % CPR
      const int j = min(panel * kTC + q / CPR, k - 1);
      rc[i] = *reinterpret_cast<const u32x4*>(
          reinterpret_cast<const unsigned char*>(Cq) + (size_t)j * d + 16 * (q % CPR));
    }
    // threads below kTC each form the key of one row r: its slot among a
    // lane's 16 accumulator values is 4 (r / 8) + r % 4
    const int jb = panel * kTC + tid;
    if (tid < kTC)
      rkey = jb < k ? bias[jb] * 16 + 15 - (4 * ((tid & 31) >> 3) + (tid & 3)) : kMasked;
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(&lc[buf][(q / CPR) * kStride + 16 * (q % CPR)]) = rc[i];
    }
    if (tid < kTC) lb[buf][tid] = rkey;
  };

  int best[kPB];  // packed 16 score + 15 - slot of the lane's best so far
  int bblk[kPB];  // first centroid of the block it came from
#pragma unroll
  for (int pb = 0; pb < kPB; ++pb) {
    best[pb] = INT32_MIN;
    bblk[pb] = -1;
  }

  gload(0);
  sstore(0);
  __syncthreads();

  // Fold a finished block (first centroid jb): packed values 32 x.q + key,
  // their maximum m, and m as the lane's best where its score part is higher.
  auto fold = [&](const i32x16* acc, const int (&kv)[16], int jb) {
#pragma unroll
    for (int pb = 0; pb < kPB; ++pb) {
      int sc[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[v] = acc[pb][v] * 32 + kv[v];
      const int m = max(max3i(max3i(sc[0], sc[1], sc[2]), max3i(sc[3], sc[4], sc[5]),
                              max3i(sc[6], sc[7], sc[8])),
                        max3i(max3i(sc[9], sc[10], sc[11]), max3i(sc[12], sc[13], sc[14]),
                              sc[15]));
      const bool up = m > (best[pb] | 15);  // a higher score, not a tie
      best[pb] = up ? m : best[pb];
      bblk[pb] = up ? jb : bblk[pb];
    }
  };

  for (int panel = 0; panel < npan; ++panel) {
    const int buf = panel & 1;
    const bool more = panel + 1 < npan;
    if (more) gload(panel + 1);
#pragma unroll
    for (int i = 0; i < kTC / 32 / CG; ++i) {
      const int cb = cg + CG * i;
      const int jb = panel * kTC + cb * 32;  // first centroid of the block (wave-uniform)
      if (jb >= k) break;                    // later blocks of the panel are past k too
      // keys of this lane's 16 centroids of the block (rows 8 g + 4 half + 0..3)
      int kv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const i32x4 b4 = *reinterpret_cast<const i32x4*>(&lb[buf][cb * 32 + 8 * g + 4 * half]);
#pragma unroll
        for (int e = 0; e < 4; ++e) kv[4 * g + e] = b4[e];
      }
      i32x16 acc[kPB];
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) acc[pb] = i32x16{};
      // A operands one k-step ahead of the MFMAs that use them
      const unsigned char* arow = &lc[buf][(cb * 32 + (lane & 31)) * kStride + 16 * half];
      u32x4 a_cur = *reinterpret_cast<const u32x4*>(arow);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 a_nxt = a_cur;
        if (ks + 1 < KS) a_nxt = *reinterpret_cast<const u32x4*>(arow + 32 * (ks + 1));
#pragma unroll
        for (int pb = 0; pb < kPB; ++pb)
          acc[pb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a_cur),
                                                          __builtin_bit_cast(i32x4, pB[pb][ks]),
                                                          acc[pb], 0, 0, 0);
        a_cur = a_nxt;
      }
      fold(acc, kv, jb);
    }
    if (more) {
      sstore(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- merge the two lanes of each point, then write --------------------------
#pragma unroll
  for (int pb = 0; pb < kPB; ++pb) {
    // unpack: score = best >> 4 (exact: the low 4 bits are 15 - slot >= 0),
    // centroid = block start + 4 half + 8 (slot / 4) + slot % 4
    int sc = best[pb] >> 4;
    const int slot = 15 - (best[pb] & 15);
    int j = bblk[pb] < 0 ? -1 : bblk[pb] + 4 * half + 8 * (slot >> 2) + (slot & 3);
    const int os = __shfl_xor(sc, 32, 64);
    const int oj = __shfl_xor(j, 32, 64);
    if (os > sc || (os == sc && (unsigned)oj < (unsigned)j)) {
      sc = os;
      j = oj;
    }
    if (half == 0) {
      const int p = pg * kTPw + pb * 32 + lane;
      m_s[cg][p] = sc;
      m_j[cg][p] = j;
      if (cg == 0) m_x[p] = xn[pb];
    }
  }
  __syncthreads();
  double dsum = 0.0;
  for (int p = tid; p < kTP; p += kThreads) {
    // merge the CG centroid subsets: highest score, lowest index on ties
    int32_t sc = m_s[0][p];
    int j = m_j[0][p];
#pragma unroll
    for (int w = 1; w < CG; ++w) {
      const int32_t s1 = m_s[w][p];
      const int j1 = m_j[w][p];
      if (s1 > sc || (s1 == sc && (unsigned)j1 < (unsigned)j)) {
        sc = s1;
        j = j1;
      }
    }
    if (j < 0 || j >= k) j = 0;  // not reachable: every point has a centroid below k
    const int slot = tile0 + p;
    if (slot < nrows) {
      const long long dist = (long long)m_x[p] - (long long)sc;  // |x - q|^2, exact
      labels[slot] = j;
      if (dists) dists[slot] = (float)dist;
      if (counts) atomicAdd(&counts[j], 1);
      dsum += (double)dist;
    }
  }
  if (obj) {
    dsum = wave_sum(dsum);
    if (lane == 0) red[wave] = dsum;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
      for (int w = 0; w < kWaves; ++w) t += red[w];
      atomicAdd(obj, t);
    }
  }
}

// Compute units of the current device, read once per device (every thread
// that races here stores the same value).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

bool assign_i8_resident_ok(int d, const void* X, const void* Cq) {
  return d % 32 == 0 && d >= 32 && d <= 256 && (uintptr_t)X % 16 == 0 &&
         (uintptr_t)Cq % 16 == 0;
}

hipError_t launch_assign_i8_resident(const void* X, int d, const uint32_t* rows, int nrows,
                                     const void* Cq, const float* bias, int k, int32_t* labels,
                                     float* dists, int32_t* counts, double* obj, bool u8,
                                     hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  const auto* x = static_cast<const uint8_t*>(X);
  const auto* c = static_cast<const int8_t*>(Cq);
  const auto* b = reinterpret_cast<const int32_t*>(bias);
  const int ks = d / 32;
  const int tpw = 32 * pblocks(ks);  // points per wave (kTPw)
  // The fewest centroid groups that still give every compute unit a
  // workgroup (one workgroup fills a CU: two waves per SIMD).
  const int cus = cu_count();
  int cgs = 1;
  while (cgs < kWaves && (nrows + tpw * (kWaves / cgs) - 1) / (tpw * (kWaves / cgs)) < cus)
    cgs *= 2;
  const int tp = tpw * (kWaves / cgs);  // points per workgroup (kTP)
  const dim3 grid((nrows + tp - 1) / tp), block(kThreads);
#define EMK_I8R_CG(KS, U8)                                                                       \
  do {                                                                                           \
    if (cgs == 1)                                                                                \
      assign_i8r_kernel<KS, U8, 1>                                                               \
          <<<grid, block, 0, st>>>(x, rows, nrows, c, b, k, labels, dists, counts, obj);         \
    else if (cgs == 2)                                                                           \
      assign_i8r_kernel<KS, U8, 2>                                                               \
          <<<grid, block, 0, st>>>(x, rows, nrows, c, b, k, labels, dists, counts, obj);         \
    else if (cgs == 4)                                                                           \
      assign_i8r_kernel<KS, U8, 4>                                                               \
          <<<grid, block, 0, st>>>(x, rows, nrows, c, b, k, labels, dists, counts, obj);         \
    else                                                                                         \
      assign_i8r_kernel<KS, U8, 8>                                                               \
          <<<grid, block, 0, st>>>(x, rows, nrows, c, b, k, labels, dists, counts, obj);         \
  } while (0)
#define EMK_I8R(KS)          \
  do {                       \
    if (u8)                  \
      EMK_I8R_CG(KS, true);  \
    else                     \
      EMK_I8R_CG(KS, false); \
  } while (0)
  switch (ks) {
    case 1: EMK_I8R(1); break;
    case 2: EMK_I8R(2); break;
    case 3: EMK_I8R(3); break;
    case 4: EMK_I8R(4); break;
    case 5: EMK_I8R(5); break;
    case 6: EMK_I8R(6); break;
    case 7: EMK_I8R(7); break;
    default: EMK_I8R(8); break;
  }
#undef EMK_I8R
#undef EMK_I8R_CG
  return hipGetLastError();
}

}  // namespace emk
