// Nearest-centroid assignment for d = 512 or 768 on gfx950 with 8-bit
// operands (int8 codes, uint8 data, FP8 E4M3 codes): points resident in
// registers, centroids streamed through LDS by the direct global-to-LDS path.
//
// Why: with both operands staged through LDS (the 64 x 64 wave tiles of the
// ring kernel) an 8-bit MFMA tile reads as many LDS bytes per clock as the LDS
// delivers, so the matrix unit and the LDS take turns. Here a wave keeps 64
// points (4 blocks of 16) as the B operands for the whole sweep (d / 16
// VGPRs per block and lane: 192 at d = 768), so each centroid fragment read
// from LDS feeds four MFMAs and the LDS runs at half its rate. One wave per
// SIMD (4 per workgroup, 256 points) leaves the registers for the points;
// the centroids come in panels of 64 rows, three panels in flight in a ring
// of LDS buffers, loaded by global_load_lds_dwordx4 (no register round trip,
// no LDS stores). Row r's 16-byte chunk c sits at chunk position c ^ (r % 16)
// of its row, so the 16 rows an MFMA operand read touches at one chunk index
// fall on 16 distinct 16-byte bank groups (d is a multiple of 256 bytes).
//
// int8 / uint8: v_mfma_i32_16x16x64_i8. Lane l holds, for row / column
// l % 16, the 16 bytes at offset 16 (l / 16) of a 64-byte k-step; the output
// puts rows 4 (l / 16) + v, v < 4, of column l % 16 in lane l. Centroids are
// the rows (M), points the columns (N).
//
// FP8: v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales. A lane holds the
// same two 16-byte pieces of a 128-byte k-step for both operands (offsets
// 16 (l / 16) and 64 + 16 (l / 16)), which are the int8 fragments of two
// consecutive 64-byte k-steps, so both kernels read the same panel layout.
//
// int8 score and fold as in the d <= 256 resident kernel: the exact integer
// score 2 x.q - |q|^2 is packed with the centroid's row in its 16-row block as
// 32 x.q + 16 bias + 15 - row (bias = -|q|^2), whose maximum over a lane's
// rows is the best score with its lowest row; a block replaces the lane's
// best only with a strictly higher score, so the first of tied maxima stays.
// |x.q| <= 128 * 127 * d < 2^24 and |q|^2 < 2^24 for d <= 1024, so packed
// values stay above -2^30 (the key of rows past k) and inside int32.
//
// uint8 rows are shifted by -128 into int8 as they are loaded; the centroid
// codes are stored shifted the same way, so every distance is unchanged.
//
// FP8 score: x.c - |c|^2 / 2 in fp32 (the bias -|c|^2 / 2 is the
// accumulator's initial value; -inf past k); the distance is |x|^2 - 2 score,
// clamped at 0. Each lane keeps, per point and per row slot v (rows 4 (l / 16)
// + v of every block), the best score so far and its block, replaced only by a
// strictly higher score, so each slot holds the first of its tied maxima; the
// slots and then the lanes are merged preferring the lower index on equal
// scores, so the lowest index of the maximum wins. A block's scores are
// folded while the next block's MFMAs run (software pipelined by one block;
// the int8 fold is short enough to run between the blocks). |x|^2 is the
// diagonal of each 16-point block's own Gram tile, one short MFMA chain
// instead of a decode and square of every byte.
#include "kernels.hpp"

namespace emk {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;            // one wave per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kNB = 4;               // 16-point blocks per wave
constexpr int kTPw = 16 * kNB;       // points per wave
constexpr int kTP = kTPw * kWaves;   // points per workgroup
constexpr int kPan = 64;             // centroid rows per panel
constexpr int kBlk = kPan / 16;      // 16-row blocks per panel
constexpr int kRing = 3;             // panels in flight
constexpr int kMasked = -(1 << 30);  // packed value of a row past k

// The direct loads of one panel of 64 centroid rows of D bytes (rows past k
// repeat row k - 1) into lc, chunk position p of row r holding the row's
// chunk p ^ (r % 16), and, from wave 0, the panel's 64 bias words into lb.
// Each wave issues kPan * D / 1024 / kWaves 1 KB loads, plus one for wave 0.
template <int D>
__device__ __forceinline__ void issue_panel(const unsigned char* C, const uint32_t* bias, int k,
                                            int panel, unsigned char* lc, uint32_t* lb, int wave,
                                            int lane) {
  constexpr int CPR = D / 16;                   // 16-byte chunks per row
  constexpr int LPW = kPan * D / 1024 / kWaves;  // 1 KB direct loads per wave
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int w = wave * LPW + i;  // 1 KB window of the panel
    const int f = w * 64 + lane;   // chunk slot in the panel
    const int r = f / CPR, p = f - (f / CPR) * CPR;
    const int j = min(panel * kPan + r, k - 1);
    lds_load16(C + (size_t)j * D + 16 * (p ^ (r & 15)), lc + w * 1024);
  }
  if (wave == 0) lds_load4(bias + min(panel * kPan + lane, k - 1), lb);
}

// Waits until this panel's loads are complete (only the next panel's may
// remain in flight: LPW windows per wave, plus the bias row for wave 0),
// then orders them before every wave's LDS reads.
template <int LPW>
__device__ __forceinline__ void wait_panel(int panel, int npan, int wave) {
  if (panel + 1 < npan) {
    EMK_WAIT_VMCNT(LPW + 1);
    if (wave != 0) EMK_WAIT_VMCNT(LPW);
  } else {
    EMK_WAIT_VMCNT(0);
  }
  lds_barrier();
}

template <int KS, bool U8>  // KS = d / 64 k-steps of 64 bytes
__global__ __launch_bounds__(kThreads, 1) void assign_i8w_kernel(
    const uint8_t* __restrict__ X, const uint32_t* __restrict__ rows, int nrows,
    const int8_t* __restrict__ Cq, const int32_t* __restrict__ bias, int k,
    int32_t* __restrict__ labels, float* __restrict__ dists, int32_t* __restrict__ counts,
    double* __restrict__ obj) {
  constexpr int d = 64 * KS;
  constexpr int PB = kPan * d;             // bytes per panel
  constexpr int LPW = PB / 1024 / kWaves;  // 1 KB direct loads per wave per panel
  static_assert(PB % (1024 * kWaves) == 0, "whole 1 KB loads per wave");
  static_assert(d % 256 == 0, "rows of whole 256-byte bank windows");
  __shared__ __attribute__((aligned(1024))) unsigned char lc[kRing][PB];
  __shared__ __attribute__((aligned(16))) int32_t lb[kRing][kPan];
  __shared__ int32_t m_s[kTP];
  __shared__ int m_j[kTP];
  __shared__ double red[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;   // the point (B) or centroid (A) row this lane feeds
  const int grp = lane >> 4;   // its 16-byte piece of each 64-byte k-step
  const int tile0 = blockIdx.x * kTP;
  const int npan = (k + kPan - 1) / kPan;
  const auto* C = reinterpret_cast<const unsigned char*>(Cq);
  const auto* B = reinterpret_cast<const uint32_t*>(bias);
  auto issue = [&](int panel, int buf) {
    issue_panel<d>(C, B, k, panel, lc[buf], reinterpret_cast<uint32_t*>(lb[buf]), wave, lane);
  };

  // ---- points of this wave into registers (B operands) ----------------------
  u32x4 pB[kNB][KS];
  int xn[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int slot = min(tile0 + wave * kTPw + nb * 16 + col, nrows - 1);
    const size_t r = rows ? (size_t)rows[slot] : (size_t)slot;
    const unsigned char* row = X + r * d + 16 * grp;
    int s = 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = *reinterpret_cast<const u32x4*>(row + 64 * ks);
      if constexpr (U8) w ^= 0x80808080u;
      pB[nb][ks] = w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int v = (int)(int8_t)(w[e] >> (8 * b));
          s += v * v;
        }
    }
    // |x|^2: the four 16-byte pieces of each k-step sit in lanes col + 16 g
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    xn[nb] = s;
  }

  int best[kNB];  // packed 32 x.q + 16 bias + 15 - row of the lane's best so far
  int bblk[kNB];  // first centroid of the block it came from
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    best[nb] = INT32_MIN;
    bblk[nb] = -1;
  }

  // A-fragment addresses: chunk (4 ks + grp) ^ col of row r = 16 blk + col
  // sits at 64 ((ks % 4) ^ (col / 4)) + 16 (grp ^ (col % 4)) + 256 (ks / 4)
  // bytes into the row (the XOR only touches the low bits), so four per-lane
  // offsets and a constant cover every k-step.
  int aoff[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
    aoff[q4] = col * d + 64 * (q4 ^ (col >> 2)) + 16 * (grp ^ (col & 3));

  issue(0, 0);
  if (npan > 1) issue(1, 1);

  for (int panel = 0; panel < npan; ++panel) {
    const int buf = panel % kRing;
    wait_panel<LPW>(panel, npan, wave);
    if (panel + 2 < npan) issue(panel + 2, (panel + 2) % kRing);
    const unsigned char* P = lc[buf];
    // Four 16-row blocks, straight-line: rows past k only carry the masked
    // key, so no block is skipped.
#pragma unroll
    for (int blk = 0; blk < kBlk; ++blk) {
      const int jb = panel * kPan + blk * 16;  // first centroid of the block
      const unsigned char* B0 = P + blk * 16 * d;
      auto afrag = [&](int ks) {
        return *reinterpret_cast<const u32x4*>(B0 + aoff[ks & 3] + 256 * (ks >> 2));
      };
      // A fragments two k-steps ahead of the MFMAs that use them
      u32x4 a0 = afrag(0), a1 = afrag(1);
      i32x4 A[kNB];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) A[nb] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 a2 = a1;
        if (ks + 2 < KS) a2 = afrag(ks + 2);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          A[nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a0),
                                                        __builtin_bit_cast(i32x4, pB[nb][ks]),
                                                        A[nb], 0, 0, 0);
        a0 = a1;
        a1 = a2;
      }
      // keys of this lane's rows 4 grp + v of the block, and the fold
      const i32x4 b4 = *reinterpret_cast<const i32x4*>(&lb[buf][blk * 16 + 4 * grp]);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        int m = INT32_MIN;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 4 * grp + v;
          const int key = jb + row < k ? b4[v] * 16 + 15 - row : kMasked;
          m = max(m, A[nb][v] * 32 + key);
        }
        const bool up = m > (best[nb] | 15);  // a higher score, not a tie
        best[nb] = up ? m : best[nb];
        bblk[nb] = up ? jb : bblk[nb];
      }
    }
  }

  // ---- merge the four lane groups of each point, then write ------------------
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    // unpack: score = best >> 4 (the low 4 bits are 15 - row >= 0)
    int sc = best[nb] >> 4;
    int j = bblk[nb] < 0 ? -1 : bblk[nb] + 15 - (best[nb] & 15);
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const int os = __shfl_xor(sc, o, 64);
      const int oj = __shfl_xor(j, o, 64);
      if (os > sc || (os == sc && (unsigned)oj < (unsigned)j)) {
        sc = os;
        j = oj;
      }
    }
    if (grp == 0) {
      const int p = wave * kTPw + nb * 16 + col;
      m_s[p] = xn[nb] - sc;  // |x - q|^2, exact
      m_j[p] = j;
    }
  }
  __syncthreads();
  double dsum = 0.0;
  for (int p = tid; p < kTP; p += kThreads) {
    const int slot = tile0 + p;
    if (slot < nrows) {
      int j = m_j[p];
      if (j < 0 || j >= k) j = 0;  // not reachable: every point has a centroid below k
      const int dist = m_s[p];
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

template <int KS>  // KS = d / 128 k-steps of 128 bytes
__global__ __launch_bounds__(kThreads, 1) void assign_f8w_kernel(
    const uint8_t* __restrict__ X, const uint32_t* __restrict__ rows, int nrows,
    const uint8_t* __restrict__ Cf, const float* __restrict__ bias, int k,
    int32_t* __restrict__ labels, float* __restrict__ dists, int32_t* __restrict__ counts,
    double* __restrict__ obj) {
  constexpr int d = 128 * KS;
  constexpr int PB = kPan * d;             // bytes per panel
  constexpr int LPW = PB / 1024 / kWaves;  // 1 KB direct loads per wave per panel
  static_assert(PB % (1024 * kWaves) == 0, "whole 1 KB loads per wave");
  static_assert(d % 256 == 0, "rows of whole 256-byte bank windows");
  __shared__ __attribute__((aligned(1024))) unsigned char lc[kRing][PB];
  __shared__ __attribute__((aligned(16))) float lb[kRing][kPan];
  __shared__ float m_s[kTP];
  __shared__ int m_j[kTP];
  __shared__ double red[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;   // the point (B) or centroid (A) row this lane feeds
  const int grp = lane >> 4;   // its two 16-byte pieces of each 128-byte k-step
  const int tile0 = blockIdx.x * kTP;
  const int npan = (k + kPan - 1) / kPan;
  const auto* B = reinterpret_cast<const uint32_t*>(bias);
  auto issue = [&](int panel, int buf) {
    issue_panel<d>(Cf, B, k, panel, lc[buf], reinterpret_cast<uint32_t*>(lb[buf]), wave, lane);
  };

  // ---- points of this wave into registers (B operands) ----------------------
  i32x8 pB[kNB][KS];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int slot = min(tile0 + wave * kTPw + nb * 16 + col, nrows - 1);
    const size_t r = rows ? (size_t)rows[slot] : (size_t)slot;
    const unsigned char* row = X + r * d + 16 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(row + 128 * ks);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(row + 128 * ks + 64);
      pB[nb][ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }
  // |x|^2 from the diagonal of each block's Gram tile: x_c . x_c sits in lane
  // 16 (c / 4) + c, slot c % 4
  float xn[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      g = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pB[nb][ks], pB[nb][ks], g, 0, 0, 0, 127,
                                                           0, 127);
    const int v = lane & 3;
    const float dg = v == 0 ? g[0] : v == 1 ? g[1] : v == 2 ? g[2] : g[3];
    xn[nb] = __shfl(dg, 16 * (col >> 2) + col, 64);
  }

  // Per lane, point block and row slot v (rows 4 grp + v of every 16-row
  // block): the best score so far and the first centroid of its block.
  f32x4 best[kNB];
  i32x4 bblk[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    best[nb] = f32x4{-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
    bblk[nb] = i32x4{-1, -1, -1, -1};
  }
  // The scores of the previous block, folded while this block's MFMAs run.
  f32x4 prev[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) prev[nb] = best[nb];
  int jprev = -1;
  auto fold_prev = [&]() {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool up = prev[nb][v] > best[nb][v];  // a higher score, not a tie
        best[nb][v] = up ? prev[nb][v] : best[nb][v];
        bblk[nb][v] = up ? jprev : bblk[nb][v];
      }
  };

  // Fragment addresses: the 128-byte k-step ks is the 64-byte k-steps 2 ks and
  // 2 ks + 1 of the int8 layout; chunk 4 h + grp of 64-byte step h sits at
  // 64 ((h % 4) ^ (col / 4)) + 16 (grp ^ (col % 4)) + 256 (h / 4) bytes into
  // row r = 16 blk + col.
  int aoff[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
    aoff[q4] = col * d + 64 * (q4 ^ (col >> 2)) + 16 * (grp ^ (col & 3));

  issue(0, 0);
  if (npan > 1) issue(1, 1);

  for (int panel = 0; panel < npan; ++panel) {
    const int buf = panel % kRing;
    wait_panel<LPW>(panel, npan, wave);
    if (panel + 2 < npan) issue(panel + 2, (panel + 2) % kRing);
    const unsigned char* P = lc[buf];
#pragma unroll
    for (int blk = 0; blk < kBlk; ++blk) {
      const int jb = panel * kPan + blk * 16;  // first centroid of the block
      const unsigned char* B0 = P + blk * 16 * d;
      auto afrag = [&](int ks) {
        const int h = 2 * ks;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(B0 + aoff[h & 3] + 256 * (h >> 2));
        const u32x4 hi =
            *reinterpret_cast<const u32x4*>(B0 + aoff[(h + 1) & 3] + 256 * ((h + 1) >> 2));
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      };
      // the accumulators start at the bias of this lane's rows 4 grp + v
      f32x4 b4 = *reinterpret_cast<const f32x4*>(&lb[buf][blk * 16 + 4 * grp]);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (jb + 4 * grp + v >= k) b4[v] = -__builtin_inff();
      i32x8 a0 = afrag(0), a1 = KS > 1 ? afrag(1) : a0;
      f32x4 A[kNB];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        i32x8 a2 = a1;
        if (ks + 2 < KS) a2 = afrag(ks + 2);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          // formats 0, 0: E4M3 operands; scales 127: 2^0
          A[nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a0, pB[nb][ks], ks == 0 ? b4 : A[nb], 0, 0, 0, 127, 0, 127);
        a0 = a1;
        a1 = a2;
      }
      // the previous block's fold, interleaved with this block's MFMAs (one
      // MFMA, then up to four VALU instructions) so that it runs while the
      // matrix core works instead of between two MFMA chains
      fold_prev();
#pragma unroll
      for (int i = 0; i < KS * kNB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // then VALU
      }
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) prev[nb] = A[nb];
      jprev = jb;
    }
  }
  fold_prev();

  // ---- merge the four lane groups of each point, then write ------------------
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    // the lane's four slots, in increasing row order within a block
    float sc = best[nb][0];
    int j = bblk[nb][0] < 0 ? -1 : bblk[nb][0] + 4 * grp;
#pragma unroll
    for (int v = 1; v < 4; ++v) {
      const float os = best[nb][v];
      const int oj = bblk[nb][v] < 0 ? -1 : bblk[nb][v] + 4 * grp + v;
      if (os > sc || (os == sc && (unsigned)oj < (unsigned)j)) {
        sc = os;
        j = oj;
      }
    }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float os = __shfl_xor(sc, o, 64);
      const int oj = __shfl_xor(j, o, 64);
      if (os > sc || (os == sc && (unsigned)oj < (unsigned)j)) {
        sc = os;
        j = oj;
      }
    }
    if (grp == 0) {
      const int p = wave * kTPw + nb * 16 + col;
      m_s[p] = fmaxf(xn[nb] - 2.0f * sc, 0.0f);  // |x - c|^2
      m_j[p] = j;
    }
  }
  __syncthreads();
  double dsum = 0.0;
  for (int p = tid; p < kTP; p += kThreads) {
    const int slot = tile0 + p;
    if (slot < nrows) {
      int j = m_j[p];
      if (j < 0 || j >= k) j = 0;  // only reachable with non-finite data
      const float dist = m_s[p];
      labels[slot] = j;
      if (dists) dists[slot] = dist;
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

}  // namespace

bool assign_i8_wide_ok(int d, const void* X, const void* Cq) {
  return (d == 512 || d == 768) && (uintptr_t)X % 16 == 0 && (uintptr_t)Cq % 16 == 0;
}

hipError_t launch_assign_i8_wide(const void* X, int d, const uint32_t* rows, int nrows,
                                 const void* Cq, const float* bias, int k, int32_t* labels,
                                 float* dists, int32_t* counts, double* obj, bool u8,
                                 hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  const auto* x = static_cast<const uint8_t*>(X);
  const auto* c = static_cast<const int8_t*>(Cq);
  const auto* b = reinterpret_cast<const int32_t*>(bias);
  const dim3 grid((nrows + kTP - 1) / kTP), block(kThreads);
#define EMK_I8W(KS)                                                                          \
  do {                                                                                       \
    if (u8)                                                                                  \
      assign_i8w_kernel<KS, true>                                                            \
          <<<grid, block, 0, st>>>(x, rows, nrows, c, b, k, labels, dists, counts, obj);     \
    else                                                                                     \
      assign_i8w_kernel<KS, false>                                                           \
          <<<grid, block, 0, st>>>(x, rows, nrows, c, b, k, labels, dists, counts, obj);     \
  } while (0)
  if (d == 512)
    EMK_I8W(8);
  else
    EMK_I8W(12);
#undef EMK_I8W
  return hipGetLastError();
}

bool assign_f8_wide_ok(int d, const void* X, const void* Cf) {
  return (d == 512 || d == 768) && (uintptr_t)X % 16 == 0 && (uintptr_t)Cf % 16 == 0;
}

hipError_t launch_assign_f8_wide(const void* X, int d, const uint32_t* rows, int nrows,
                                 const void* Cf, const float* bias, int k, int32_t* labels,
                                 float* dists, int32_t* counts, double* obj, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  const auto* x = static_cast<const uint8_t*>(X);
  const auto* c = static_cast<const uint8_t*>(Cf);
  const dim3 grid((nrows + kTP - 1) / kTP), block(kThreads);
  if (d == 512)
    assign_f8w_kernel<4><<<grid, block, 0, st>>>(x, rows, nrows, c, bias, k, labels, dists,
                                                 counts, obj);
  else
    assign_f8w_kernel<6><<<grid, block, 0, st>>>(x, rows, nrows, c, bias, k, labels, dists,
                                                 counts, obj);
  return hipGetLastError();
}

}  // namespace emk
