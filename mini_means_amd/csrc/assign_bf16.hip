// Nearest-centroid assignment for bf16 or fp16 data of small dimension
// (d = 16 * KS, d <= 128) on gfx950: points resident in registers, centroids
// streamed. The two 16-bit formats differ only in the decode of |x|^2 and in
// the MFMA (v_mfma_f32_32x32x16_bf16 or _f16, same operand layout).
//
// At d = 128 a bf16 point row is 256 bytes, so a wave can keep 96 points as
// MFMA B operands in registers (96 VGPRs) for the whole sweep over the
// centroids, and the only streamed data are the bf16 centroid panels, shared
// by the eight waves of the workgroup through LDS (two waves per SIMD, so one
// wave's argmax work overlaps the other's MFMAs). Each centroid fragment read
// from LDS feeds three MFMAs, and it is read one k-step ahead of them (a
// whole block ahead would not fit the registers beside 96 points; deeper
// lookahead measured no faster). v_mfma_f32_32x32x16_bf16
// tiles put 32 centroids on M and 32 points on N: after the KS k-steps each
// lane holds 16 centroid scores x.c - |c|^2/2 (the bias is the accumulator's
// initial value) of one point. The argmax first reduces the 16 scores to
// their maximum; only when some lane of the wave improves on its running best
// does the wave walk the 16 scores in index order to record which centroid it
// was (after the first panels such improvements are rare). Ties keep the
// first strict maximum per lane and the lower index when lanes merge.
#include "kernels.hpp"

namespace emk {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kPB = 3;                  // 32-point blocks per wave (96 points resident)
constexpr int kWaves = 8;               // two waves per SIMD: one folds while the other multiplies
constexpr int kThreads = 64 * kWaves;
constexpr int kTPw = 32 * kPB;          // points per wave
constexpr int kTP = kTPw * kWaves;      // points per workgroup
constexpr int kTC = 256;                // centroids per LDS panel
constexpr int kRowB = 256;              // LDS row slab: a whole centroid row (d <= 128)
constexpr int kStride = kRowB + 16;     // 16 consecutive rows hit 16 disjoint 4-bank groups

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

template <int KS, bool F16>
__global__ __launch_bounds__(kThreads, 1) void assign_bf16_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ rows, int nrows,
    const uint16_t* __restrict__ Chat, const float* __restrict__ bias, int k,
    int32_t* __restrict__ labels, float* __restrict__ dists, int32_t* __restrict__ counts,
    double* __restrict__ obj, int sim) {
  constexpr int d = 16 * KS;
  constexpr int CPR = d * 2 / 16;              // 16-byte chunks per centroid row
  constexpr int PER = kTC * CPR / kThreads;    // chunk loads per thread per panel
  __shared__ __attribute__((aligned(16))) unsigned char lc[2][kTC * kStride];
  __shared__ float lb[2][kTC];
  __shared__ float m_s[2][kTP];
  __shared__ int m_j[2][kTP];
  __shared__ double red[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;  // which 8 of each 16-element k-step this lane holds
  const int tile0 = blockIdx.x * kTP;

  // ---- points of this wave into registers (B operands) ----------------------
  u32x4 pB[kPB][KS];
  float xn[kPB];
#pragma unroll
  for (int pb = 0; pb < kPB; ++pb) {
    const int slot = min(tile0 + wave * kTPw + pb * 32 + (lane & 31), nrows - 1);
    const size_t r = rows ? (size_t)rows[slot] : (size_t)slot;
    const unsigned char* row = reinterpret_cast<const unsigned char*>(X + r * d);
    float s = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      pB[pb][ks] = *reinterpret_cast<const u32x4*>(row + 32 * ks + 16 * half);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = pB[pb][ks][e];
        const float lo = half_to_f32((uint16_t)(w & 0xFFFFu), F16);
        const float hi = half_to_f32((uint16_t)(w >> 16), F16);
        s += lo * lo + hi * hi;
      }
    }
    xn[pb] = s + __shfl_xor(s, 32, 64);
  }

  // ---- centroid panel staging ------------------------------------------------
  const int npan = (k + kTC - 1) / kTC;
  u32x4 rc[PER];
  float rbias = 0.0f;
  auto gload = [&](int panel) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + kThreads * i;  // chunk id: row q / CPR, chunk q % CPR
      const int j = min(panel * kTC + q / CPR, k - 1);
      rc[i] = *reinterpret_cast<const u32x4*>(
          reinterpret_cast<const unsigned char*>(Chat + (size_t)j * d) + 16 * (q % CPR));
    }
    const int jb = panel * kTC + tid;  // threads below kTC load one bias each
    if (tid < kTC) rbias = jb < k ? bias[jb] : -__builtin_inff();
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(&lc[buf][(q / CPR) * kStride + 16 * (q % CPR)]) = rc[i];
    }
    if (tid < kTC) lb[buf][tid] = rbias;
  };

  float best[kPB];
  int bidx[kPB];
#pragma unroll
  for (int pb = 0; pb < kPB; ++pb) {
    best[pb] = -__builtin_inff();
    bidx[pb] = -1;
  }

  gload(0);
  sstore(0);
  __syncthreads();

  // Fold a finished block into the running best: the max m of the 16 scores
  // per point; only when some lane of the wave improves on its best does the
  // wave locate, on those lanes, the first of the 16 slots holding m (slots
  // are in increasing centroid order: row 8 * (v / 4) + (v % 4) + 4 * half),
  // which is the lowest-index maximum, as an ordered strict-> walk finds.
  auto fold = [&](const f32x16* acc, int base) {
    float m[kPB];
    bool imp[kPB];
#pragma unroll
    for (int pb = 0; pb < kPB; ++pb) {
      const f32x16 c = acc[pb];
      m[pb] = fmaxf(max3f(max3f(c[0], c[1], c[2]), max3f(c[3], c[4], c[5]),
                          max3f(c[6], c[7], c[8])),
                    max3f(max3f(c[9], c[10], c[11]), max3f(c[12], c[13], c[14]), c[15]));
      imp[pb] = m[pb] > best[pb];
    }
#pragma unroll
    for (int pb = 0; pb < kPB; ++pb) {
      if (__builtin_amdgcn_ballot_w64(imp[pb])) {
        const f32x16 c = acc[pb];
        int v0 = 15;
#pragma unroll
        for (int v = 14; v >= 0; --v) v0 = c[v] == m[pb] ? v : v0;
        if (imp[pb]) {
          best[pb] = m[pb];
          bidx[pb] = base + 8 * (v0 >> 2) + (v0 & 3);
        }
      }
    }
  };

  for (int panel = 0; panel < npan; ++panel) {
    const int buf = panel & 1;
    const bool more = panel + 1 < npan;
    if (more) gload(panel + 1);
    // biases of a block's 32 centroids (the accumulators' initial values) and
    // the row of its A operands
    auto block_init = [&](int cb) {
      f32x16 init;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 b4 = *reinterpret_cast<const float4*>(&lb[buf][cb * 32 + 8 * g + 4 * half]);
        init[4 * g + 0] = b4.x;
        init[4 * g + 1] = b4.y;
        init[4 * g + 2] = b4.z;
        init[4 * g + 3] = b4.w;
      }
      return init;
    };
    auto block_row = [&](int cb) {
      return &lc[buf][(cb * 32 + (lane & 31)) * kStride + 16 * half];
    };
    f32x16 init = block_init(0);
    u32x4 a_cur = *reinterpret_cast<const u32x4*>(block_row(0));
#pragma unroll
    for (int cb = 0; cb < kTC / 32; ++cb) {
      f32x16 acc[kPB];
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) acc[pb] = init;
      // A operands one k-step ahead of the MFMAs that use them; during the
      // last k-step, the next block's first operands and its biases
      const unsigned char* arow = block_row(cb);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 a_nxt = a_cur;
        if (ks + 1 < KS) {
          a_nxt = *reinterpret_cast<const u32x4*>(arow + 32 * (ks + 1));
        } else if (cb + 1 < kTC / 32) {
          a_nxt = *reinterpret_cast<const u32x4*>(block_row(cb + 1));
          init = block_init(cb + 1);
        }
        // keep these reads above this step's MFMAs (the scheduler would
        // otherwise sink them to just before their first use)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pb = 0; pb < kPB; ++pb) {
          if constexpr (F16)
            acc[pb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a_cur),
                                                             __builtin_bit_cast(f16x8, pB[pb][ks]),
                                                             acc[pb], 0, 0, 0);
          else
            acc[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a_cur), __builtin_bit_cast(bf16x8, pB[pb][ks]), acc[pb],
                0, 0, 0);
        }
        a_cur = a_nxt;
      }
      fold(acc, panel * kTC + cb * 32 + 4 * half);
    }
    if (more) {
      sstore(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- merge the two lanes of each point, then write --------------------------
#pragma unroll
  for (int pb = 0; pb < kPB; ++pb) {
    float sc = best[pb];
    int j = bidx[pb];
    const float os = __shfl_xor(sc, 32, 64);
    const int oj = __shfl_xor(j, 32, 64);
    if (os > sc || (os == sc && (unsigned)oj < (unsigned)j)) {
      sc = os;
      j = oj;
    }
    if (half == 0) {
      m_s[0][wave * kTPw + pb * 32 + lane] = sc;
      m_j[0][wave * kTPw + pb * 32 + lane] = j;
      m_s[1][wave * kTPw + pb * 32 + lane] = xn[pb];
    }
  }
  __syncthreads();
  double dsum = 0.0;
  for (int p = tid; p < kTP; p += kThreads) {
    int j = m_j[0][p];
    if (j < 0 || j >= k) j = 0;  // only reachable with non-finite data
    const int slot = tile0 + p;
    if (slot < nrows) {
      // sim (spherical e-means): similarity out, error 2 - 2 x similarity
      const float dist = fmaxf(m_s[1][p] - 2.0f * m_s[0][p], 0.0f);
      labels[slot] = j;
      if (dists) dists[slot] = sim ? m_s[0][p] : dist;
      if (counts) atomicAdd(&counts[j], 1);
      dsum += sim ? 2.0 - 2.0 * (double)m_s[0][p] : (double)dist;
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

}  // namespace

bool assign_bf16_resident_ok(int d, const void* X, const void* Chat) {
  return (d == 32 || d == 64 || d == 96 || d == 128) && (uintptr_t)X % 16 == 0 &&
         (uintptr_t)Chat % 16 == 0;
}

hipError_t launch_assign_bf16_resident(const void* X, int d, const uint32_t* rows, int nrows,
                                       const void* Chat, const float* bias, int k,
                                       int32_t* labels, float* dists, int32_t* counts,
                                       double* obj, bool sim, bool f16, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  const dim3 grid((nrows + kTP - 1) / kTP), block(kThreads);
  const auto* x = static_cast<const uint16_t*>(X);
  const auto* c = static_cast<const uint16_t*>(Chat);
  const int sm = sim ? 1 : 0;
#define EMK_RES(KS)                                                                           \
  do {                                                                                        \
    if (f16)                                                                                  \
      assign_bf16_kernel<KS, true>                                                            \
          <<<grid, block, 0, st>>>(x, rows, nrows, c, bias, k, labels, dists, counts, obj, sm); \
    else                                                                                      \
      assign_bf16_kernel<KS, false>                                                           \
          <<<grid, block, 0, st>>>(x, rows, nrows, c, bias, k, labels, dists, counts, obj, sm); \
  } while (0)
  switch (d) {
    case 32:
      EMK_RES(2);
      break;
    case 64:
      EMK_RES(4);
      break;
    case 96:
      EMK_RES(6);
      break;
    default:
      EMK_RES(8);
      break;
  }
#undef EMK_RES
  return hipGetLastError();
}

}  // namespace emk
