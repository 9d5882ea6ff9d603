// Radix-select building blocks shared by the top-K and merge kernels.
#pragma once

#include "dsa_common.h"

namespace dsa {

constexpr int kBins = 2048;  // 11-bit digits (the last key digit has 10 bits)

struct Bucket {
  uint32_t bin;    // chosen bin
  uint32_t need;   // how many elements still to take from it
  uint32_t count;  // how many elements it holds
};

// Walks a histogram of `nbins` bins from the top bin down (DESC) or from bin
// 0 up (!DESC) and finds the bin in which the running count reaches `need`.
// Every thread of the block must call it; on return every thread sees the
// same result.  `scan` holds >= NT/64 + 1 words, `res` 3 words of LDS.
template <int NT, bool DESC>
__device__ Bucket find_bucket(const uint32_t* hist, int nbins, uint32_t need,
                              uint32_t* scan, uint32_t* res) {
  constexpr int kPer = kBins / NT;  // bins per thread (nbins <= kBins)
  const int t = threadIdx.x;
  uint32_t c[kPer];
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int d = t * kPer + q;  // rank of the bin in walking order
    const int bin = DESC ? nbins - 1 - d : d;
    c[q] = d < nbins ? hist[bin] : 0u;
    sum += c[q];
  }
  uint32_t total;
  uint32_t before = block_excl_scan<NT>(sum, scan, total);
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int d = t * kPer + q;
    if (d < nbins && before < need && before + c[q] >= need) {
      res[0] = (uint32_t)(DESC ? nbins - 1 - d : d);
      res[1] = need - before;
      res[2] = c[q];
    }
    before += c[q];
  }
  __syncthreads();
  Bucket b{res[0], res[1], res[2]};
  __syncthreads();  // res may be rewritten by the next call
  return b;
}

template <int NT>
__device__ __forceinline__ void clear_hist(uint32_t* hist, int n) {
  for (int i = threadIdx.x; i < n; i += NT) hist[i] = 0u;
}

}  // namespace dsa
