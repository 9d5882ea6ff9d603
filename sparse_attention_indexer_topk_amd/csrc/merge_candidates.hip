// Stable global top-K over the gathered (score, global id) candidates.
//
// What is computed (PR #46076 report, 实现拆解 item 1, and the selector call
// of `_merge_dcp_topk_global` in 关键源码片段): among a row's valid
// candidates, the k best under (larger score, then smaller global id); the
// output lists their ids in ascending order followed by -1.
//
// How (one workgroup per row):
//  1. stage the candidates' order keys in LDS (invalid ones get a key no
//     score can have) and count the valid ones while building the first
//     11-bit histogram;
//  2. radix-select the threshold score key exactly as the top-K kernel does;
//  3. if more candidates share the threshold key than are needed, radix
//     select among them on the id (ascending, 3 x 8 bits), which makes the
//     (score, id) order total without a 64-bit sort;
//  4. collect the selected ids and emit them in ascending order through an
//     LDS bitmap over the id space (16 KB per 2^17 ids; larger id ranges are
//     swept chunk by chunk), a popcount scan giving each id its slot.
#include "launchers.h"
#include "select_common.h"

namespace dsa {

constexpr int kMergeThreads = 512;
constexpr int kMergeCap = 16384;        // candidate keys staged in LDS (64 KB)
constexpr int kIdChunk = 1 << 17;       // ids covered by one bitmap sweep
constexpr uint32_t kInvalidKey = 0xffffffffu;  // above every real key (max 0xff800000)
constexpr int kMaxK = 2048;

template <bool STAGED>
__global__ __launch_bounds__(kMergeThreads) void merge_candidates_kernel(
    const float2* __restrict__ cand, int n_cand, int k, int id_bound, int* __restrict__ ids) {
  constexpr int NT = kMergeThreads;
  __shared__ uint32_t s_keys[STAGED ? kMergeCap : 1];
  __shared__ uint32_t s_hist[kBins];
  __shared__ uint32_t s_bitmap[kIdChunk / 32];
  __shared__ int s_list[kMaxK];
  __shared__ uint32_t s_scan[NT / kWave + 1];
  __shared__ uint32_t s_res[4];
  __shared__ uint32_t s_nvalid;
  __shared__ uint32_t s_nlist;

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const float2* src = cand + (int64_t)row * n_cand;
  int* out = ids + (int64_t)row * k;

  auto cand_key = [&](const float2 c) -> uint32_t {
    const float id = c.y;
    const bool valid = id >= 0.0f && id < (float)id_bound;  // false for NaN
    return valid ? order_key(__float_as_uint(c.x)) : kInvalidKey;
  };
  auto key_at = [&](int i) -> uint32_t {
    if constexpr (STAGED) return s_keys[i];
    else return cand_key(src[i]);
  };
  auto id_at = [&](int i) -> int { return (int)src[i].y; };

  // ---- 1. stage keys, count valid, first histogram ------------------------
  clear_hist<NT>(s_hist, kBins);
  if (tid == 0) { s_nvalid = 0; s_nlist = 0; }
  __syncthreads();
  uint32_t my_valid = 0;
  for (int i = tid; i < n_cand; i += NT) {
    const uint32_t key = cand_key(src[i]);
    if constexpr (STAGED) s_keys[i] = key;
    if (key != kInvalidKey) {
      ++my_valid;
      atomicAdd(&s_hist[key >> 21], 1u);
    }
  }
  if (my_valid) atomicAdd(&s_nvalid, my_valid);
  __syncthreads();
  const uint32_t n_valid = s_nvalid;

  // ---- 2/3. threshold (score key, then id among equal keys) ---------------
  uint32_t prefix = 0;
  int shift = 32;        // shift == 32: every valid candidate is selected
  bool tie_by_id = false;
  uint32_t id_thr = 0;   // with tie_by_id: take equal keys with id <= id_thr
  if (n_valid > (uint32_t)k) {
    Bucket bk = find_bucket<NT, true>(s_hist, kBins, (uint32_t)k, s_scan, s_res);
    prefix = bk.bin;
    shift = 21;
    if (bk.count != bk.need) {
      clear_hist<NT>(s_hist, kBins);
      __syncthreads();
      for (int i = tid; i < n_cand; i += NT) {
        const uint32_t key = key_at(i);
        if (key != kInvalidKey && (key >> 21) == prefix)
          atomicAdd(&s_hist[(key >> 10) & 0x7ffu], 1u);
      }
      __syncthreads();
      bk = find_bucket<NT, true>(s_hist, kBins, bk.need, s_scan, s_res);
      prefix = (prefix << 11) | bk.bin;
      shift = 10;
      if (bk.count != bk.need) {
        clear_hist<NT>(s_hist, 1024);
        __syncthreads();
        for (int i = tid; i < n_cand; i += NT) {
          const uint32_t key = key_at(i);
          if (key != kInvalidKey && (key >> 10) == prefix) atomicAdd(&s_hist[key & 0x3ffu], 1u);
        }
        __syncthreads();
        bk = find_bucket<NT, true>(s_hist, 1024, bk.need, s_scan, s_res);
        prefix = (prefix << 10) | bk.bin;
        shift = 0;
        if (bk.count != bk.need) {
          // equal full keys: take the `need` smallest ids (ids < 2^24)
          tie_by_id = true;
          uint32_t need = bk.need;
          uint32_t id_prefix = 0;
          for (int level = 0; level < 3; ++level) {
            const int ishift = 16 - 8 * level;
            clear_hist<NT>(s_hist, 256);
            __syncthreads();
            for (int i = tid; i < n_cand; i += NT) {
              if (key_at(i) != prefix) continue;
              const uint32_t id = (uint32_t)id_at(i);
              if (level == 0 || (id >> (ishift + 8)) == id_prefix)
                atomicAdd(&s_hist[(id >> ishift) & 0xffu], 1u);
            }
            __syncthreads();
            Bucket ib = find_bucket<NT, false>(s_hist, 256, need, s_scan, s_res);
            id_prefix = (id_prefix << 8) | ib.bin;
            need = ib.need;
          }
          id_thr = id_prefix;  // exactly one candidate has this id
        }
      }
    }
  }

  // ---- 4a. collect the selected ids ----------------------------------------
  for (int i = tid; i < n_cand; i += NT) {
    const uint32_t key = key_at(i);
    if (key == kInvalidKey) continue;
    bool sel;
    if (shift == 32) {
      sel = true;
    } else {
      const uint32_t p = key >> shift;
      sel = p > prefix;
      if (p == prefix) sel = !tie_by_id || (uint32_t)id_at(i) <= id_thr;
    }
    if (sel) {
      const uint32_t slot = atomicAdd(&s_nlist, 1u);
      if (slot < (uint32_t)kMaxK) s_list[slot] = id_at(i);
    }
  }
  __syncthreads();
  uint32_t n_list = s_nlist;
  if (n_list > (uint32_t)k) n_list = (uint32_t)k;

  // ---- 4b. ascending-id output through the bitmap ---------------------------
  constexpr int kWords = kIdChunk / 32;
  constexpr int kWpt = kWords / NT;  // words per thread
  uint32_t written = 0;
  for (int c0 = 0; c0 < id_bound; c0 += kIdChunk) {
    for (int w = tid; w < kWords; w += NT) s_bitmap[w] = 0u;
    __syncthreads();
    for (int i = tid; i < (int)n_list; i += NT) {
      const int id = s_list[i];
      if (id >= c0 && id < c0 + kIdChunk) {
        const int off = id - c0;
        atomicOr(&s_bitmap[off >> 5], 1u << (off & 31));
      }
    }
    __syncthreads();
    uint32_t words[kWpt];
    uint32_t cnt = 0;
#pragma unroll
    for (int q = 0; q < kWpt; ++q) {
      words[q] = s_bitmap[tid * kWpt + q];
      cnt += __popc(words[q]);
    }
    uint32_t total;
    uint32_t pos = written + block_excl_scan<NT>(cnt, s_scan, total);
#pragma unroll
    for (int q = 0; q < kWpt; ++q) {
      uint32_t w = words[q];
      while (w) {
        const int b = __ffs(w) - 1;
        w &= w - 1;
        if (pos < (uint32_t)k) out[pos] = c0 + (tid * kWpt + q) * 32 + b;
        ++pos;
      }
    }
    written += total;
    if (written >= n_list) break;  // uniform: total is block-wide
  }
  for (int i = (int)n_list + tid; i < k; i += NT) out[i] = -1;
}

int launch_merge_candidates(const float* cand, int rows, int n_cand, int k, int id_bound,
                            int* ids, hipStream_t stream) {
  const float2* c2 = reinterpret_cast<const float2*>(cand);
  if (n_cand <= kMergeCap) {
    hipLaunchKernelGGL(merge_candidates_kernel<true>, dim3(rows), dim3(kMergeThreads), 0,
                       stream, c2, n_cand, k, id_bound, ids);
  } else {
    hipLaunchKernelGGL(merge_candidates_kernel<false>, dim3(rows), dim3(kMergeThreads), 0,
                       stream, c2, n_cand, k, id_bound, ids);
  }
  return 0;
}

}  // namespace dsa
