// Stable global top-K over the gathered (score, global id) candidates.
//
// What is computed (PR #46076 report, 实现拆解 item 1, and the selector call
// of `_merge_dcp_topk_global` in 关键源码片段): among a row's valid
// candidates, the k best under (larger score, then smaller global id); the
// output lists their ids in ascending order followed by -1.
//
// How (one workgroup of 1024 threads per row):
//  1. every thread holds E candidates (interleaved 16-byte loads of
//     candidate pairs) as (order key, id) in registers; E = 8 or 16 holds rows
//     of up to 8K / 16K candidates, longer rows are swept in chunks that every
//     pass re-reads from L2;
//  2. the k-th best score key kt comes from the same two steps as in the
//     top-K kernel: a histogram on bins linear in the score, then an exact
//     rank of the few keys in the threshold bin (radix select on the keys
//     when that bin is crowded);
//  3. when fewer kt-scored candidates are taken than exist, the smallest ids
//     among them win: their ids are ranked the same way (radix select on the
//     ids, 3 x 8 bits, when there are many), which makes (score, id) a total
//     order without a sort;
//  4. the selected ids set bits of an LDS bitmap over the id range (32 KB per
//     2^18 ids; larger ranges are swept piecewise); each thread owns a run of
//     bitmap words and a popcount scan gives each set bit its output slot;
//     the ids are staged in LDS and leave in one coalesced write, -1 after.
#include "launchers.h"
#include "select_common.h"

namespace dsa {

constexpr int kMergeThreads = 1024;
constexpr int kMergeMaxK = 2048;
constexpr int kMergeListCap = 128;
constexpr int kIdChunk = 1 << 18;   // ids covered by one bitmap sweep
constexpr int kIdWords = kIdChunk / 32;
constexpr int kIdWordsPerThread = kIdWords / kMergeThreads;
constexpr uint32_t kInvalidKey = 0xffffffffu;  // above every real key (max 0xff800000)

struct MergeSmem {
  uint32_t hist[2][kBins];
  uint32_t bitmap[kIdWords];
  int stage[kMergeMaxK];
  uint32_t list[kMergeListCap];
  float red[2 * (kMergeThreads / kWave)];
  uint32_t scan[kMergeThreads / kWave];
  uint32_t res[4];
  uint32_t cnt;
  uint32_t nvalid;
};

// order key -> fp32 bits; exact except that -0 comes back as +0 and every
// NaN as one NaN, neither of which changes a bin or a comparison
__device__ __forceinline__ uint32_t key_to_bits(uint32_t key) {
  return (key & 0x80000000u) ? (key ^ 0x80000000u) : ~key;
}

template <int E, bool RESIDENT>
__device__ __forceinline__ void merge_row(MergeSmem& sm, const float* __restrict__ src,
                                          int n_cand, int k, int id_bound, bool vec,
                                          int* __restrict__ out) {
  constexpr int NT = kMergeThreads;
  constexpr int kChunk = NT * E;
  const int tid = threadIdx.x;
  const int nchunks = RESIDENT ? 1 : (n_cand + kChunk - 1) / kChunk;

  uint32_t key[E];
  int id[E];
  // slot e of chunk c0 is candidate c0 + 2 * (tid + NT * (e / 2)) + e % 2
  auto load = [&](int c0) {
#pragma unroll
    for (int v = 0; v < E / 2; ++v) {
      const int i = c0 + 2 * (tid + NT * v);
      float4 x = make_float4(0.f, -1.f, 0.f, -1.f);
      if (vec) {
        if (i < n_cand) x = *reinterpret_cast<const float4*>(src + 2 * (int64_t)i);  // n_cand even
      } else {
        if (i < n_cand) {
          const float2 a = *reinterpret_cast<const float2*>(src + 2 * (int64_t)i);
          x.x = a.x;
          x.y = a.y;
        }
        if (i + 1 < n_cand) {
          const float2 b = *reinterpret_cast<const float2*>(src + 2 * (int64_t)(i + 1));
          x.z = b.x;
          x.w = b.y;
        }
      }
      const bool ok0 = x.y >= 0.0f && x.y < (float)id_bound;   // false for NaN
      const bool ok1 = x.w >= 0.0f && x.w < (float)id_bound;
      key[2 * v] = ok0 ? order_key(__float_as_uint(x.x)) : kInvalidKey;
      key[2 * v + 1] = ok1 ? order_key(__float_as_uint(x.z)) : kInvalidKey;
      id[2 * v] = ok0 ? (int)x.y : -1;
      id[2 * v + 1] = ok1 ? (int)x.w : -1;
    }
  };
  auto sweep = [&](auto f) {
    for (int c = 0; c < nchunks; ++c) {
      if (!RESIDENT) load(c * kChunk);
      f();
    }
  };

  // ---- 1. valid count, min / max of the finite valid scores ---------------
  if (RESIDENT) load(0);
  float vmin = INFINITY, vmax = -INFINITY;
  uint32_t my_valid = 0;
  sweep([&]() {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ok = key[e] != kInvalidKey;
      const uint32_t bits = key_to_bits(key[e]);
      const bool fin = ok && finite_bits(bits);
      my_valid += ok ? 1u : 0u;
      vmin = fminf(vmin, fin ? __uint_as_float(bits) : INFINITY);
      vmax = fmaxf(vmax, fin ? __uint_as_float(bits) : -INFINITY);
    }
  });
  clear_words<NT>(sm.hist[0], kBins);
  {   // the first bitmap sweep's words, cleared here behind the loads
    const int span0 = id_bound < kIdChunk ? id_bound : kIdChunk;
    for (int w = tid; w < (span0 + 31) >> 5; w += NT) sm.bitmap[w] = 0u;
  }
  if (tid == 0) {
    sm.cnt = 0;
    sm.nvalid = 0;
  }
  __syncthreads();
  {
    const uint32_t w = wave_scan_incl(my_valid);
    if (lane_id() == kWave - 1 && w) atomicAdd(&sm.nvalid, w);
  }
  block_min_max<NT>(vmin, vmax, sm.red);
  const uint32_t n_valid = sm.nvalid;
  const LinBins lb = make_lin_bins(vmin, vmax);

  // ---- 2/3. threshold: score key, then id among equal keys ---------------
  bool take_all = true;   // every valid candidate is selected
  uint32_t kt = 0;        // otherwise: keys above kt, ...
  bool tie_by_id = false; // ... and kt-keyed ones, all or those with id <= id_thr
  uint32_t id_thr = 0;
  if (n_valid > (uint32_t)k) {
    take_all = false;
    sweep([&]() {
#pragma unroll
      for (int e = 0; e < E; ++e)
        atomicAdd(&sm.hist[0][lin_bin(key_to_bits(key[e]), lb)], key[e] != kInvalidKey ? 1u : 0u);
    });
    __syncthreads();
    const Bucket bk = block_find_bucket<true>(sm.hist[0], kBins, (uint32_t)k, sm.res);
    uint32_t take, n_kt;
    if (bk.count <= (uint32_t)kMergeListCap) {
      sweep([&]() {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (key[e] != kInvalidKey && lin_bin(key_to_bits(key[e]), lb) == bk.bin) {
            const uint32_t slot = atomicAdd(&sm.cnt, 1u);
            sm.list[slot] = key[e];   // slot < count <= the list capacity
          }
        }
      });
      __syncthreads();
      list_threshold<NT>(sm.list, (int)bk.count, bk.need, sm.res);
      kt = sm.res[0];
      take = sm.res[1];
      n_kt = sm.res[2];
      __syncthreads();   // res and the list are reused below
    } else {
      radix_threshold<NT>(sm.hist, sm.res, (uint32_t)k, [&](auto f) {
        sweep([&]() {
#pragma unroll
          for (int e = 0; e < E; ++e) f(key[e], key[e] != kInvalidKey);
        });
      }, &kt, &take, &n_kt);
    }
    if (take < n_kt) {
      // the `take` smallest ids among the kt-keyed candidates (distinct ids)
      tie_by_id = true;
      if (n_kt <= (uint32_t)kMergeListCap) {
        if (tid == 0) sm.cnt = 0;
        __syncthreads();
        sweep([&]() {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            if (key[e] == kt) {
              const uint32_t slot = atomicAdd(&sm.cnt, 1u);
              sm.list[slot] = (uint32_t)id[e];
            }
          }
        });
        __syncthreads();
        list_kth_smallest<NT>(sm.list, (int)n_kt, take, &sm.res[3]);
        id_thr = sm.res[3];
      } else {
        uint32_t need = take, id_prefix = 0;
        for (int level = 0; level < 3; ++level) {
          const int ishift = 16 - 8 * level;
          clear_words<NT>(sm.hist[0], 256);
          __syncthreads();
          sweep([&]() {
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const uint32_t u = (uint32_t)id[e];
              if (key[e] == kt && (level == 0 || (u >> (ishift + 8)) == id_prefix))
                atomicAdd(&sm.hist[0][(u >> ishift) & 0xffu], 1u);
            }
          });
          __syncthreads();
          const Bucket ib = block_find_bucket<false>(sm.hist[0], 256, need, sm.res);
          id_prefix = (id_prefix << 8) | ib.bin;
          need = ib.need;
          __syncthreads();   // res and the histogram are rewritten next level
        }
        id_thr = id_prefix;   // ids < 2^24: three digits cover them
      }
    }
  }
  const uint32_t n_sel = n_valid < (uint32_t)k ? n_valid : (uint32_t)k;

  // ---- 4. ascending-id output through the bitmap --------------------------
  auto selected = [&](int e) {
    if (key[e] == kInvalidKey) return false;
    if (take_all || key[e] > kt) return true;
    return key[e] == kt && (!tie_by_id || (uint32_t)id[e] <= id_thr);
  };
  uint32_t written = 0;
  for (int b0 = 0; b0 < id_bound && written < n_sel; b0 += kIdChunk) {
    const int span = (id_bound - b0) < kIdChunk ? (id_bound - b0) : kIdChunk;
    const int nwords = (span + 31) >> 5;
    const int wpt = (nwords + NT - 1) / NT;   // words per thread, <= kIdWordsPerThread
    if (b0 > 0) {   // later sweeps clear the words the previous sweep used
      for (int w = tid; w < nwords; w += NT) sm.bitmap[w] = 0u;
      __syncthreads();
    }
    sweep([&]() {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int off = id[e] - b0;
        if (off >= 0 && off < span && selected(e))
          atomicOr(&sm.bitmap[off >> 5], 1u << (off & 31));
      }
    });
    __syncthreads();
    uint32_t words[kIdWordsPerThread];
    uint32_t cnt = 0;
#pragma unroll
    for (int q = 0; q < kIdWordsPerThread; ++q) {
      const int w = tid * wpt + q;
      words[q] = (q < wpt && w < nwords) ? sm.bitmap[w] : 0u;
      cnt += __popc(words[q]);
    }
    uint32_t total;
    uint32_t pos = written + block_scan_excl<NT>(cnt, sm.scan, total);
#pragma unroll
    for (int q = 0; q < kIdWordsPerThread; ++q) {
      uint32_t w = words[q];
      while (w) {
        const int b = __builtin_ctz(w);
        w &= w - 1;
        if (pos < (uint32_t)k) sm.stage[pos] = b0 + (tid * wpt + q) * 32 + b;
        ++pos;
      }
    }
    written += total;
  }
  __syncthreads();
  const int n_out = (int)(written < (uint32_t)k ? written : (uint32_t)k);
  for (int i = tid; i < k; i += NT) out[i] = i < n_out ? sm.stage[i] : -1;
}

template <int E>
__global__ __launch_bounds__(kMergeThreads) void merge_candidates_kernel(
    const float* __restrict__ cand, int n_cand, int k, int id_bound, int* __restrict__ ids,
    int vec) {
  __shared__ MergeSmem sm;
  const int row = blockIdx.x;
  const float* src = cand + (int64_t)row * n_cand * 2;
  int* out = ids + (int64_t)row * k;
  if (n_cand <= kMergeThreads * E)
    merge_row<E, true>(sm, src, n_cand, k, id_bound, vec != 0, out);
  else
    merge_row<E, false>(sm, src, n_cand, k, id_bound, vec != 0, out);
}

int launch_merge_candidates(const float* cand, int rows, int n_cand, int k, int id_bound,
                            int* ids, hipStream_t stream) {
  const int vec = ((uintptr_t)cand % 16 == 0 && n_cand % 2 == 0) ? 1 : 0;
  if (n_cand <= kMergeThreads * 8)
    hipLaunchKernelGGL((merge_candidates_kernel<8>), dim3(rows), dim3(kMergeThreads), 0, stream,
                       cand, n_cand, k, id_bound, ids, vec);
  else
    hipLaunchKernelGGL((merge_candidates_kernel<16>), dim3(rows), dim3(kMergeThreads), 0,
                       stream, cand, n_cand, k, id_bound, ids, vec);
  return 0;
}

}  // namespace dsa
