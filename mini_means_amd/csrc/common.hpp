// Device-side building blocks shared by the e-means kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace emk {

constexpr int kWave = 64;

// Random streams (distinct Philox counter words).
constexpr uint64_t kStreamInit = 1;
constexpr uint64_t kStreamPerm = 2;
constexpr uint64_t kStreamRevive = 3;
constexpr uint64_t kStreamSign = 4;

// ---------------------------------------------------------------------------
// Philox4x64-10, Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3" (SC'11): ten rounds of two 64x64->128 multiplies, key bumped by
// the Weyl increments between rounds.
// ---------------------------------------------------------------------------
struct U64x4 {
  uint64_t w0, w1, w2, w3;
};

__host__ __device__ __forceinline__ uint64_t mulhi64(uint64_t a, uint64_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __umul64hi(a, b);
#else
  return (uint64_t)(((unsigned __int128)a * b) >> 64);
#endif
}

__host__ __device__ __forceinline__ U64x4 philox(uint64_t c0, uint64_t c1, uint64_t c2,
                                                 uint64_t c3, uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t lo0 = kM0 * c0, hi0 = mulhi64(kM0, c0);
    const uint64_t lo1 = kM1 * c2, hi1 = mulhi64(kM1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return {c0, c1, c2, c3};
}

// ---------------------------------------------------------------------------
// Keyed permutation of [0, n): balanced 4-round Feistel network on 2h bits
// with Philox as round function (Luby-Rackoff), cycle-walked onto [0, n)
// (Black-Rogaway). Every pass draws a fresh order with its own pass word.
// ---------------------------------------------------------------------------
struct PermKey {
  uint64_t n, seed, stream, pass;
  uint32_t h;
  uint64_t mask;
};

inline PermKey make_perm_key(uint64_t n, uint64_t seed, uint64_t stream, uint64_t pass) {
  uint32_t m = 0;
  while (m < 64 && ((n - 1) >> m)) ++m;
  uint32_t h = (m + 1) / 2;
  if (h < 1) h = 1;
  PermKey k{n, seed, stream, pass, h, (h >= 64) ? ~0ull : ((1ull << h) - 1)};
  return k;
}

__host__ __device__ __forceinline__ uint64_t feistel(uint64_t v, const PermKey& k) {
  uint64_t L = v >> k.h, R = v & k.mask;
#pragma unroll
  for (uint64_t r = 0; r < 4; ++r) {
    const uint64_t f = philox(R, r, k.pass, k.stream, k.seed, 0).w0 & k.mask;
    const uint64_t nl = R;
    R = L ^ f;
    L = nl;
  }
  return (L << k.h) | R;
}

__host__ __device__ __forceinline__ uint64_t perm_at(uint64_t i, const PermKey& k) {
  uint64_t v = feistel(i, k);
  while (v >= k.n) v = feistel(v, k);
  return v;
}

// 53 random bits in [0, 1) for the revival draw of dead cluster j at step t.
__device__ __forceinline__ double revive_uniform(uint64_t seed, uint64_t t, uint64_t j) {
  const U64x4 w = philox(j, t, 0, kStreamRevive, seed, 0);
  return (double)(w.w0 >> 11) * 0x1.0p-53;
}

// Sign (+1 / -1) of coordinate e for the split at step t that refills j.
__device__ __forceinline__ float split_sign(uint64_t seed, uint64_t t, uint64_t j, uint32_t e) {
  const U64x4 w = philox(j, t, e >> 8, kStreamSign, seed, 0);
  const uint32_t q = (e >> 6) & 3;
  const uint64_t word = q == 0 ? w.w0 : q == 1 ? w.w1 : q == 2 ? w.w2 : w.w3;
  return ((word >> (e & 63)) & 1) ? -1.0f : 1.0f;
}

// ---------------------------------------------------------------------------
// bf16 storage
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// IEEE binary16 storage: the hardware conversion rounds to nearest, ties to
// even, keeps subnormals and overflows to infinity (finite range +-65504).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Search copy of a centroid coordinate in bf16 (f16 false) or fp16 bits.
__device__ __forceinline__ uint16_t to_half_rne(float f, bool f16) {
  return f16 ? f32_to_f16_rne(f) : f32_to_bf16_rne(f);
}

__device__ __forceinline__ float half_to_f32(uint16_t h, bool f16) {
  return f16 ? f16_to_f32(h) : bf16_to_f32(h);
}

// FP8 E4M3 (OCP): sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
// exponent 0 holds the subnormals m * 2^-9; 0x7F / 0xFF are NaN; no
// infinities; the largest finite value is 448.
//
// Decoding: the 7 low bits placed at fp32 bit 20 read as 2^(e-127) (1 + m/8)
// for e >= 1 and as the fp32 subnormal m 2^-129 for e = 0; one exact product
// by 2^120 gives 2^(e-7) (1 + m/8) and m 2^-9 (fp32 denormals are kept). The
// NaN codes, which no encoder here produces, decode to +-480.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  return __uint_as_float(((c & 0x80u) << 24) | ((c & 0x7Fu) << 20)) * 0x1p120f;
}

// Nearest E4M3 value (ties to the even mantissa), saturating at +-448; the
// sign of a zero result follows x. Non-finite input is not supported.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  if (a < 0x1p-6f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);  // 8 = 2^-6, the first normal
  uint32_t b = __float_as_uint(a);
  b += 0x7FFFFu + ((b >> 20) & 1u);  // round the fp32 mantissa to 3 bits, ties to even
  return sign | (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
}

// ---------------------------------------------------------------------------
// reductions
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const T o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// Inclusive scan across the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const T o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Inclusive scan across a block of NT threads (NT a multiple of 64, <= 1024).
// `tmp` must hold NT/64 elements of shared memory. Ends with a barrier.
template <typename T, int NT>
__device__ __forceinline__ T block_incl_scan(T v, T* tmp) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_incl_scan(v);
  if (lane == kWave - 1) tmp[w] = v;
  __syncthreads();
  if (w == 0) {
    T t = lane < NT / kWave ? tmp[lane] : T(0);
    t = wave_incl_scan(t);
    if (lane < NT / kWave) tmp[lane] = t;
  }
  __syncthreads();
  if (w > 0) v += tmp[w - 1];
  __syncthreads();
  return v;
}

template <typename T, int NT>
__device__ __forceinline__ T block_sum(T v, T* tmp) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_sum(v);
  if (lane == 0) tmp[w] = v;
  __syncthreads();
  T t = T(0);
  for (int i = 0; i < NT / kWave; ++i) t += tmp[i];
  __syncthreads();
  return t;
}

// ---------------------------------------------------------------------------
// fp64 wave scan on DPP lane moves (no LDS round trip): row shifts 1, 2, 4, 8
// scan each row of 16 lanes, then row broadcasts 15 and 31 carry the row
// totals across the wave. Lanes outside a move's source range add zero.
// ---------------------------------------------------------------------------
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_move_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  int lo = (int)(uint32_t)b, hi = (int)(uint32_t)(b >> 32);
  lo = __builtin_amdgcn_update_dpp(0, lo, CTRL, ROWMASK, 0xF, false);
  hi = __builtin_amdgcn_update_dpp(0, hi, CTRL, ROWMASK, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

__device__ __forceinline__ double wave_scan_f64(double v) {
  v += dpp_move_f64<0x111, 0xF>(v);  // row_shr:1
  v += dpp_move_f64<0x112, 0xF>(v);  // row_shr:2
  v += dpp_move_f64<0x114, 0xF>(v);  // row_shr:4
  v += dpp_move_f64<0x118, 0xF>(v);  // row_shr:8
  v += dpp_move_f64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_move_f64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// ---------------------------------------------------------------------------
// Direct global-to-LDS loads (gfx950 global_load_lds_dword / _dwordx4).
// One wave-wide load: lane i's 16 (or 4) bytes at src go to LDS bytes
// [lds + 16 i, lds + 16 i + 16) (or 4 i ...); lds must be wave-uniform.
// Written as asm so that the compiler does not treat every later LDS read as
// aliasing the load (it would wait for all loads in flight before each one);
// the asm has no register outputs, and completion is waited for with
// EMK_WAIT_VMCNT. M0 is clobbered: the backend reserves it and sets it right
// before any instruction that reads it, so no value of its own is live
// across the asm.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr_t;

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_load16(const void* src, void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(const void* src, void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(m0), "v"(src)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding).
#define EMK_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Workgroup barrier that orders LDS accesses only. __syncthreads() also
// orders global memory, which waits for every load in flight, direct loads
// of later panels or stages included; their completion is waited for
// explicitly.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace emk
