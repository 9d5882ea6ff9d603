// Device helpers shared by the DSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kWave = 64;
constexpr int kLatent = 576;
constexpr int kValue = 512;
constexpr int kRope = 64;

// ---------------------------------------------------------------- keys ----
// Order-preserving map fp32 -> uint32: a > b (as numbers) iff key(a) > key(b).
// -0.0 is folded onto +0.0 (they tie), every NaN maps to 0 (below -inf).
__device__ __forceinline__ uint32_t order_key(uint32_t bits) {
  if (bits == 0x80000000u) bits = 0u;
  if ((bits & 0x7fffffffu) > 0x7f800000u) return 0u;
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

// ---------------------------------------------------- shard index maps ----
// Global token t lives on shard (t / I) % S at local position
// (t / (I*S)) * I + t % I; shard r's local position l is global token
// ((l / I) * S + r) * I + l % I.
__device__ __forceinline__ int owner_of(int t, int S, int I) { return (t / I) % S; }
__device__ __forceinline__ int local_of(int t, int S, int I) {
  return (t / (I * S)) * I + t % I;
}
__device__ __forceinline__ int global_of(int r, int l, int S, int I) {
  return ((l / I) * S + r) * I + l % I;
}
// Number of the global tokens 0 .. n-1 that shard r holds.
__host__ __device__ __forceinline__ int local_count(int n, int r, int S, int I) {
  const int period = I * S;
  int rem = n % period - r * I;
  rem = rem < 0 ? 0 : (rem > I ? I : rem);
  return (n / period) * I + rem;
}

// ------------------------------------------------------------ scans ------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    uint32_t t = __shfl_up(v, d, kWave);
    if (lane >= d) v += t;
  }
  return v;
}

// Exclusive prefix sum across the block; returns this thread's prefix and
// the block total.  `scratch` holds >= NW + 1 words of LDS.  Contains the
// barriers it needs; every thread of the block must call it.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch,
                                                    uint32_t& total) {
  constexpr int NW = NT / kWave;
  const int wave = threadIdx.x / kWave;
  const uint32_t incl = wave_incl_scan(v);
  if (lane_id() == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t s = scratch[w];
    before += (w < wave) ? s : 0u;
    all += s;
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

// Max / sum across groups of lanes that share (lane % 16) — used to reduce
// over the four 16-lane groups of a wave.
__device__ __forceinline__ float max_over_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, kWave));
  v = fmaxf(v, __shfl_xor(v, 32, kWave));
  return v;
}
__device__ __forceinline__ float sum_over_groups(float v) {
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}

// -------------------------------------------------------------- formats ---
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// fp32 -> fp8 e4m3 (OCP "fn": bias 7, no inf, max 448), nearest even,
// saturating finite values at +-448, NaN -> 0x7f; the sign is kept (also for
// results that round to zero).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t s = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return 0x7fu;
  if (a > 448.0f) return s | 0x7eu;
  if (a < 0.015625f) {                      // below 2^-6: subnormal grid 2^-9
    const uint32_t m = (uint32_t)rintf(a * 512.0f);  // 0..8, 8 = 2^-6
    return s | m;
  }
  uint32_t ua = __float_as_uint(a);
  ua += 0x7ffffu + ((ua >> 20) & 1u);       // round away 20 fraction bits
  const int e = (int)(ua >> 23) - 127;      // -6 .. 8
  const uint32_t m = (ua >> 20) & 7u;
  return s | ((uint32_t)(e + 7) << 3) | m;
}

}  // namespace dsa
