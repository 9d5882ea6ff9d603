// Per-shard stable top-K over fp32 indexer logits with the (score, global id)
// candidate pack fused into its epilogue.
//
// What is computed (PR #46076 report, 关键源码片段 `_merge_dcp_topk_global`
// and 实现拆解 item 1): for every row and every shard, the k best local
// positions of the row's valid local range, best = larger logit, ties by
// smaller position; then each selection becomes a (score, global_id) pair in
// the shard's k columns of the gathered candidate buffer.
//
// How (one workgroup per (row, shard)):
//  1. stream the row's valid logits from HBM with 16-byte loads into LDS
//     (raw bits), building a 2048-bin histogram of the top 11 bits of the
//     order-preserving key on the way;
//  2. walk the histogram from the top to find the bin holding the k-th key;
//     refine inside that bin with the next 11, then the last 10 key bits
//     (each refinement re-reads LDS only) until the bin is either taken
//     whole or the exact k-th key is known;
//  3. one stable pass in position order: element e is selected when its key
//     prefix is above the threshold prefix, or equal to it and among the
//     first `need` such elements; a block-wide exclusive scan of packed
//     (above, equal) counts gives every selection its output slot, so the
//     output is in ascending position with no sort and no atomics.
// Rows whose valid range holds <= k positions take everything (no select).
#include "launchers.h"
#include "select_common.h"

namespace dsa {

constexpr int kTopkThreads = 512;
constexpr int kTopkCap = 16384;  // logits staged in LDS (64 KB)
constexpr int kTopkIpt = 4;      // elements per thread per compaction tile

template <bool STAGED>
__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(
    const float* __restrict__ logits, int64_t ld, int64_t shard_stride, int rows,
    int ctx, const int* __restrict__ row_starts, const int* __restrict__ row_ends,
    int k, int S, int I, int shard_first, int* __restrict__ local_idx,
    float* __restrict__ cand, int vec4) {
  constexpr int NT = kTopkThreads;
  __shared__ __attribute__((aligned(16))) uint32_t s_vals[STAGED ? kTopkCap : 4];
  __shared__ uint32_t s_hist[kBins];
  __shared__ uint32_t s_scan[NT / kWave + 1];
  __shared__ uint32_t s_res[4];

  const int row = blockIdx.x;
  const int j = blockIdx.y;
  const int r = shard_first + j;
  const int tid = threadIdx.x;
  const float* src = logits + (int64_t)j * shard_stride + (int64_t)row * ld;

  int gs = row_starts ? row_starts[row] : 0;
  int ge = row_ends ? row_ends[row] : ctx;
  gs = gs < 0 ? 0 : (gs > ctx ? ctx : gs);
  ge = ge < gs ? gs : (ge > ctx ? ctx : ge);
  const int lo = local_count(gs, r, S, I);
  const int hi = local_count(ge, r, S, I);
  const int n = hi - lo;

  int* oidx = local_idx ? local_idx + ((int64_t)j * rows + row) * k : nullptr;
  float2* ocand =
      cand ? reinterpret_cast<float2*>(cand) + ((int64_t)row * S + r) * k : nullptr;

  auto emit = [&](int pos, int l, uint32_t bits) {
    if (oidx) oidx[pos] = l;
    if (ocand) ocand[pos] = make_float2(__uint_as_float(bits), (float)global_of(r, l, S, I));
  };

  if (n <= k) {  // everything valid is selected
    for (int i = tid; i < k; i += NT) {
      if (i < n) {
        emit(i, lo + i, __float_as_uint(src[lo + i]));
      } else {
        if (oidx) oidx[i] = -1;
        if (ocand) ocand[i] = make_float2(-INFINITY, -1.0f);
      }
    }
    return;
  }

  auto val = [&](int i) -> uint32_t {
    if constexpr (STAGED) return s_vals[i];
    else return __float_as_uint(src[lo + i]);
  };

  // ---- 1. stage + first-digit histogram ---------------------------------
  clear_hist<NT>(s_hist, kBins);
  __syncthreads();
  if (STAGED && vec4) {
    const float4* src4 = reinterpret_cast<const float4*>(src);
    for (int v = (lo >> 2) + tid; (v << 2) < hi; v += NT) {
      const float4 x = src4[v];
      const uint32_t b[4] = {__float_as_uint(x.x), __float_as_uint(x.y),
                             __float_as_uint(x.z), __float_as_uint(x.w)};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = (v << 2) + q;
        if (e >= lo && e < hi) {
          if constexpr (STAGED) s_vals[e - lo] = b[q];
          atomicAdd(&s_hist[order_key(b[q]) >> 21], 1u);
        }
      }
    }
  } else {
    for (int i = tid; i < n; i += NT) {
      const uint32_t b = __float_as_uint(src[lo + i]);
      if constexpr (STAGED) s_vals[i] = b;
      atomicAdd(&s_hist[order_key(b) >> 21], 1u);
    }
  }
  __syncthreads();

  // ---- 2. find the threshold prefix --------------------------------------
  Bucket bk = find_bucket<NT, true>(s_hist, kBins, (uint32_t)k, s_scan, s_res);
  uint32_t prefix = bk.bin;
  int shift = 21;
  if (bk.count != bk.need) {
    clear_hist<NT>(s_hist, kBins);
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t key = order_key(val(i));
      if ((key >> 21) == prefix) atomicAdd(&s_hist[(key >> 10) & 0x7ffu], 1u);
    }
    __syncthreads();
    bk = find_bucket<NT, true>(s_hist, kBins, bk.need, s_scan, s_res);
    prefix = (prefix << 11) | bk.bin;
    shift = 10;
    if (bk.count != bk.need) {
      clear_hist<NT>(s_hist, 1024);
      __syncthreads();
      for (int i = tid; i < n; i += NT) {
        const uint32_t key = order_key(val(i));
        if ((key >> 10) == prefix) atomicAdd(&s_hist[key & 0x3ffu], 1u);
      }
      __syncthreads();
      bk = find_bucket<NT, true>(s_hist, 1024, bk.need, s_scan, s_res);
      prefix = (prefix << 10) | bk.bin;
      shift = 0;
    }
  }
  const uint32_t need = bk.need;

  // ---- 3. stable compaction in position order ----------------------------
  constexpr int kTile = NT * kTopkIpt;
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < n; base += kTile) {
    const int e0 = base + tid * kTopkIpt;
    uint32_t bits[kTopkIpt];
    bool loaded = false;
    if constexpr (STAGED) {
      if (e0 + kTopkIpt <= n) {
        const uint4 v4 = *reinterpret_cast<const uint4*>(&s_vals[e0]);
        bits[0] = v4.x; bits[1] = v4.y; bits[2] = v4.z; bits[3] = v4.w;
        loaded = true;
      }
    }
    if (!loaded) {
#pragma unroll
      for (int q = 0; q < kTopkIpt; ++q) bits[q] = (e0 + q < n) ? val(e0 + q) : 0u;
    }
    uint32_t gt = 0, eq = 0;
    uint32_t pk[kTopkIpt];
#pragma unroll
    for (int q = 0; q < kTopkIpt; ++q) {
      pk[q] = order_key(bits[q]) >> shift;
      const bool in = e0 + q < n;
      gt += (in && pk[q] > prefix) ? 1u : 0u;
      eq += (in && pk[q] == prefix) ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t excl = block_excl_scan<NT>(gt | (eq << 16), s_scan, total);
    uint32_t g_before = run_gt + (excl & 0xffffu);
    uint32_t e_before = run_eq + (excl >> 16);
#pragma unroll
    for (int q = 0; q < kTopkIpt; ++q) {
      if (e0 + q >= n) break;
      if (pk[q] > prefix) {
        const uint32_t pos = g_before + (e_before < need ? e_before : need);
        if (pos < (uint32_t)k) emit((int)pos, lo + e0 + q, bits[q]);
        ++g_before;
      } else if (pk[q] == prefix) {
        if (e_before < need) {
          const uint32_t pos = g_before + e_before;
          if (pos < (uint32_t)k) emit((int)pos, lo + e0 + q, bits[q]);
        }
        ++e_before;
      }
    }
    run_gt += total & 0xffffu;
    run_eq += total >> 16;
  }
}

int launch_topk_select(const float* logits, int64_t ld, int64_t shard_stride, int rows,
                       int ctx, const int* row_starts, const int* row_ends, int k,
                       int S, int I, int shard_first, int shard_count, int* local_idx,
                       float* cand, hipStream_t stream) {
  const int max_local = local_count(ctx, shard_first, S, I);
  const bool vec4 = ((uintptr_t)logits % 16 == 0) && (ld % 4 == 0) && (shard_stride % 4 == 0);
  dim3 grid(rows, shard_count);
  if (max_local <= kTopkCap) {
    hipLaunchKernelGGL(topk_select_kernel<true>, grid, dim3(kTopkThreads), 0, stream, logits,
                       ld, shard_stride, rows, ctx, row_starts, row_ends, k, S, I,
                       shard_first, local_idx, cand, vec4 ? 1 : 0);
  } else {
    hipLaunchKernelGGL(topk_select_kernel<false>, grid, dim3(kTopkThreads), 0, stream, logits,
                       ld, shard_stride, rows, ctx, row_starts, row_ends, k, S, I,
                       shard_first, local_idx, cand, vec4 ? 1 : 0);
  }
  return 0;
}

}  // namespace dsa
