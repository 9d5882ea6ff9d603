// Radix-select building blocks shared by the top-K, merge and convert kernels.
#pragma once

#include "dsa_common.h"

namespace dsa {

constexpr int kBins = 2048;  // 11-bit digits (the last key digit has 10 bits)

struct Bucket {
  uint32_t bin;    // chosen bin
  uint32_t need;   // how many elements still to take from it
  uint32_t count;  // how many elements it holds
};

// ---------------------------------------------------------------- DPP ------
// DPP controls of the gfx9 family (wave64): row_shr:n shifts within a 16-lane
// row, row_bcast:15 / row_bcast:31 carry a row's last lane into the next rows.
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes of a wave (uint32, wrapping), built
// from DPP row shifts and row broadcasts — no LDS round trips.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr1, 0xf, 0xf, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr2, 0xf, 0xf, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr4, 0xf, 0xf, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr8, 0xf, 0xf, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast15, 0xa, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast31, 0xc, 0xf, false);
  return v;
}

// Block-wide exclusive prefix sum: a DPP wave scan, the wave totals through
// LDS (`scratch`, >= NT/64 words) and one barrier.  Returns the thread's
// exclusive prefix and the block total.  Every thread must call it; the
// caller must not rewrite `scratch` before a later barrier.
template <int NT>
__device__ __forceinline__ uint32_t block_scan_excl(uint32_t v, uint32_t* scratch,
                                                    uint32_t& total) {
  constexpr int NW = NT / kWave;
  const int wave = threadIdx.x / kWave;
  const uint32_t incl = wave_scan_incl(v);
  if (lane_id() == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t s = scratch[w];
    before += (w < wave) ? s : 0u;
    all += s;
  }
  total = all;
  return before + incl - v;
}

// Finds, in a histogram of `nbins` (a multiple of 64, at most 2048) bins, the
// bin where the running count, walked from the top bin down (DESC) or from
// bin 0 up (!DESC), reaches `need`.  Runs in ONE wave: each lane sums a
// contiguous run of bins, a DPP scan locates the owning lane, then the lanes
// scan that run.  The caller publishes the result through LDS.
template <bool DESC>
__device__ __forceinline__ Bucket wave_find_bucket(const uint32_t* hist, int nbins,
                                                   uint32_t need) {
  const int lane = lane_id();
  const int per = nbins / kWave;                       // bins per lane (<= 32)
  auto bin_of = [&](int rank) { return DESC ? nbins - 1 - rank : rank; };
  uint32_t sum = 0;
  for (int j = 0; j < per; ++j) {
    const int r = lane * per + ((j + lane) & (per - 1));   // rotated: fewer bank conflicts
    sum += hist[bin_of(r)];
  }
  const uint32_t incl = wave_scan_incl(sum);
  const uint32_t before = incl - sum;
  const uint64_t hit = __ballot(before < need && incl >= need);
  // need <= the histogram's total, so some lane holds it; the guard keeps a
  // corrupted count from indexing past the histogram
  const int owner = hit ? (int)__builtin_ctzll(hit) : kWave - 1;
  const uint32_t ob = (uint32_t)__builtin_amdgcn_readlane((int)before, owner);
  const uint32_t c = lane < per ? hist[bin_of(owner * per + lane)] : 0u;
  const uint32_t ci = wave_scan_incl(c);
  const uint64_t hit2 = __ballot(lane < per && ob + ci - c < need && ob + ci >= need);
  const int j = hit2 ? (int)__builtin_ctzll(hit2) : per - 1;
  const uint32_t cj = (uint32_t)__builtin_amdgcn_readlane((int)c, j);
  const uint32_t cij = (uint32_t)__builtin_amdgcn_readlane((int)ci, j);
  Bucket b;
  b.bin = (uint32_t)bin_of(owner * per + j);
  b.need = need - (ob + cij - cj);
  b.count = cj;
  return b;
}

// Wave 0 finds the bucket and publishes it in `res` (3 words of LDS); after
// the barrier every thread reads it.  The histogram must be complete (a
// barrier between its last update and this call).
template <bool DESC>
__device__ __forceinline__ Bucket block_find_bucket(const uint32_t* hist, int nbins, uint32_t need,
                                                    uint32_t* res) {
  if (threadIdx.x < kWave) {
    const Bucket b = wave_find_bucket<DESC>(hist, nbins, need);
    if (threadIdx.x == 0) {
      res[0] = b.bin;
      res[1] = b.need;
      res[2] = b.count;
    }
  }
  __syncthreads();
  return Bucket{res[0], res[1], res[2]};
}

template <int NT>
__device__ __forceinline__ void clear_words(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += NT) p[i] = 0u;
}

// ------------------------------------------------ linear score bins -------
// First-pass bins that are linear in the score between the row's smallest and
// largest finite valid score: unlike the top bits of the order key (which
// group by binary exponent, so that typical logits crowd into a dozen bins)
// they spread the scores evenly, and the bin holding the k-th best score
// usually holds only a handful of elements.  The map is monotone in the
// score order of order_key (NaN and -inf in bin 0, +inf in the last bin;
// finite scores through a rounded fused subtract and a multiply, both
// monotone), so "bin above b" implies "key above every key of bin b".
struct LinBins {
  float lo_half;  // smallest finite score / 2 (0 when there is none)
  float scale;    // bins per unit of (score / 2): finite and > 0
};

__device__ __forceinline__ LinBins make_lin_bins(float vmin, float vmax) {
  LinBins lb{0.f, 1.f};
  if (vmin <= vmax) {   // at least one finite score
    lb.lo_half = vmin * 0.5f;
    const float range = vmax * 0.5f - lb.lo_half;  // halves: no overflow
    if (range > 0.f) lb.scale = fminf((float)kBins / range, 3.0e38f);   // tiny range: fewer bins
  }
  return lb;
}

// (score/2 - lo_half) * scale, clamped to the table.  Special values need no
// branch: fmaxf(NaN, 0) is 0, so NaN lands in bin 0 with -inf, and +inf in
// the last bin, where their order keys rank; the map is monotone in the
// score, so a bin above b only holds keys above every key of bin b.  Any
// other value (a slot outside the valid range, counted with weight 0) is
// clamped into the table.
__device__ __forceinline__ uint32_t lin_bin(uint32_t bits, LinBins lb) {
  const float t = __builtin_fmaf(__uint_as_float(bits), 0.5f, -lb.lo_half) * lb.scale;
  return (uint32_t)fminf(fmaxf(t, 0.f), (float)(kBins - 1));
}

__device__ __forceinline__ bool finite_bits(uint32_t bits) {
  return (bits & 0x7f800000u) != 0x7f800000u;
}

// Max over the 64 lanes of a wave, left in every lane: DPP row shifts and
// row broadcasts build an inclusive max-scan (lanes outside a row read
// -inf), lane 63 holds the wave's max.
__device__ __forceinline__ float wave_max(float v) {
  const int ninf = __float_as_int(-INFINITY);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), kDppRowShr1, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), kDppRowShr2, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), kDppRowShr4, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), kDppRowShr8, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), kDppRowBcast15, 0xa, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), kDppRowBcast31, 0xc, 0xf, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// Min and max over the block; `scratch` holds 2 * NT/64 floats.  One barrier.
template <int NT>
__device__ __forceinline__ void block_min_max(float& vmin, float& vmax, float* scratch) {
  constexpr int NW = NT / kWave;
  vmax = wave_max(vmax);
  vmin = -wave_max(-vmin);
  const int wave = threadIdx.x / kWave;
  if (lane_id() == 0) {
    scratch[wave] = vmin;
    scratch[NW + wave] = vmax;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    vmin = fminf(vmin, scratch[w]);
    vmax = fmaxf(vmax, scratch[NW + w]);
  }
}

// Exact threshold among the `c` (<= 128) order keys in `list`: the
// `need`-th largest key kt, how many elements equal to kt are taken (need
// minus the keys above kt), and how many keys equal kt.  Wave 0 holds the
// list in its lanes (two keys per lane) and compares every pair through
// readlane broadcasts; the lane holding a key with (#keys above) < need <=
// (#keys at or above) publishes the result (several such lanes hold the same
// kt and write the same words).  One barrier; the result is in res[0] (kt),
// res[1] (take) and res[2] (how many keys equal kt).
template <int NT>
__device__ __forceinline__ void list_threshold(const uint32_t* list, int c, uint32_t need,
                                               uint32_t* res) {
  if (threadIdx.x < kWave) {
    const int lane = lane_id();
    const uint32_t k0 = lane < c ? list[lane] : 0u;
    const uint32_t k1 = lane + kWave < c ? list[lane + kWave] : 0u;
    uint32_t a0 = 0, g0 = 0, a1 = 0, g1 = 0;   // above / at-least counts of k0 and k1
    for (int j = 0; j < c; ++j) {
      const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane(
          (int)(j < kWave ? k0 : k1), j & (kWave - 1));
      a0 += kj > k0 ? 1u : 0u;
      g0 += kj >= k0 ? 1u : 0u;
      a1 += kj > k1 ? 1u : 0u;
      g1 += kj >= k1 ? 1u : 0u;
    }
    if (lane < c && a0 < need && need <= g0) {
      res[0] = k0;
      res[1] = need - a0;
      res[2] = g0 - a0;
    }
    if (lane + kWave < c && a1 < need && need <= g1) {
      res[0] = k1;
      res[1] = need - a1;
      res[2] = g1 - a1;
    }
  }
  __syncthreads();
}

// The `kth`-smallest (1-based) of the `c` (<= 128) DISTINCT values in
// `list`, written to *res by the lane holding it; wave 0 compares all pairs
// through readlane broadcasts.  One barrier.
template <int NT>
__device__ __forceinline__ void list_kth_smallest(const uint32_t* list, int c, uint32_t kth,
                                                  uint32_t* res) {
  if (threadIdx.x < kWave) {
    const int lane = lane_id();
    const uint32_t v0 = lane < c ? list[lane] : 0u;
    const uint32_t v1 = lane + kWave < c ? list[lane + kWave] : 0u;
    uint32_t b0 = 0, b1 = 0;   // how many values lie below v0 / v1
    for (int j = 0; j < c; ++j) {
      const uint32_t vj = (uint32_t)__builtin_amdgcn_readlane(
          (int)(j < kWave ? v0 : v1), j & (kWave - 1));
      b0 += vj < v0 ? 1u : 0u;
      b1 += vj < v1 ? 1u : 0u;
    }
    if (lane < c && b0 + 1 == kth) *res = v0;
    if (lane + kWave < c && b1 + 1 == kth) *res = v1;
  }
  __syncthreads();
}

// Radix select of the `need`-th largest key over all valid elements, 11/11/10
// bits (the fallback when a linear bin is crowded, e.g. all scores equal).
// `for_keys(f)` calls f(key, valid) for every element of the block's row.
// Returns kt, how many kt-equal elements to take, and how many there are.
// Uses both histograms; ends with a barrier, so `res` and the histograms may
// be reused afterwards.
template <int NT, typename ForKeys>
__device__ __forceinline__ void radix_threshold(uint32_t (*hist)[kBins], uint32_t* res,
                                                uint32_t need, ForKeys for_keys, uint32_t* kt,
                                                uint32_t* take, uint32_t* n_kt) {
  clear_words<NT>(hist[0], kBins);
  clear_words<NT>(hist[1], kBins);
  __syncthreads();
  for_keys([&](uint32_t key, bool ok) {
    if (ok) atomicAdd(&hist[0][key >> 21], 1u);
  });
  __syncthreads();
  Bucket bk = block_find_bucket<true>(hist[0], kBins, need, res);
  uint32_t prefix = bk.bin;
  for_keys([&](uint32_t key, bool ok) {
    if (ok && (key >> 21) == prefix) atomicAdd(&hist[1][(key >> 10) & 0x7ffu], 1u);
  });
  clear_words<NT>(hist[0], 1024);
  __syncthreads();
  bk = block_find_bucket<true>(hist[1], kBins, bk.need, res);
  prefix = (prefix << 11) | bk.bin;
  for_keys([&](uint32_t key, bool ok) {
    if (ok && (key >> 10) == prefix) atomicAdd(&hist[0][key & 0x3ffu], 1u);
  });
  __syncthreads();
  bk = block_find_bucket<true>(hist[0], 1024, bk.need, res);
  *kt = (prefix << 10) | bk.bin;
  *take = bk.need;
  *n_kt = bk.count;
  __syncthreads();
}

}  // namespace dsa
