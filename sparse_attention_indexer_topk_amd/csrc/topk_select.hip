// Per-shard stable top-K over fp32 indexer logits with the (score, global id)
// candidate pack fused into its epilogue.
//
// What is computed (PR #46076 report, 关键源码片段 `_merge_dcp_topk_global`
// and 实现拆解 item 1): for every row and every shard, the k best local
// positions of the row's valid local range, best = larger logit, ties by
// smaller position; then each selection becomes a (score, global_id) pair in
// the shard's k columns of the gathered candidate buffer.
//
// How (one workgroup of 1024 threads per (row, shard)):
//  1. thread t holds E contiguous logits of the row in registers (16-byte
//     loads) with their order keys; E = 8 or 16 holds rows of up to 8K / 16K
//     local positions, longer rows are swept in chunks of 1024*E that every
//     pass re-reads from L2;
//  2. the k-th best key kt is found in two steps: a 2048-bin histogram on
//     bins linear in the score between the row's min and max finite score
//     (one wave finds the bin b where the count from the top reaches k), then
//     the few keys of bin b are listed in LDS and ranked exactly; a bin too
//     full to rank falls back to an 11/11/10-bit radix select on the keys;
//  3. one stable pass in position order: an element is taken when its key is
//     above kt, or equal to it and among the first `take` such elements; a
//     block exclusive scan of packed (above, equal) counts gives each
//     selection its output slot — ascending position, no sort, no atomics
//     deciding order.  Selections are staged in LDS and written out
//     coalesced.
// Rows whose valid range holds <= k positions take everything.
#include "launchers.h"
#include "select_common.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkMaxK = 2048;
constexpr int kTopkListCap = 128;   // threshold-bin keys ranked directly

struct TopkSmem {
  uint32_t hist[2][kBins];
  uint32_t list[kTopkListCap];
  float2 out[kTopkMaxK];
  int idx[kTopkMaxK];
  float red[2 * (kTopkThreads / kWave)];
  uint32_t scan[2][kTopkThreads / kWave];
  uint32_t res[4];
  uint32_t cnt;
};

template <int E, bool RESIDENT>
__device__ __forceinline__ void topk_row(TopkSmem& sm, const float* __restrict__ src, int lo,
                                         int hi, bool vec, int k, int S, int I, int r,
                                         int* __restrict__ oidx, float2* __restrict__ ocand,
                                         bool out_vec, const uint32_t* pre) {
  constexpr int NT = kTopkThreads;
  constexpr int kChunk = NT * E;
  const int tid = threadIdx.x;
  // pre: the thread's E logits from local position tid*E on, already loaded
  // (the whole shard row fits one chunk), so the row starts at position 0
  const int base = pre ? 0 : (vec ? (lo & ~3) : lo);
  const int nchunks = RESIDENT ? 1 : (hi - base + kChunk - 1) / kChunk;

  uint32_t raw[E], key[E];
  uint32_t vmask = 0;   // bit e: element e lies in [lo, hi)
  auto load = [&](int c0) {
    const int p0 = c0 + tid * E;
    if (pre) {
#pragma unroll
      for (int e = 0; e < E; ++e) raw[e] = pre[e];
    } else if (vec) {
#pragma unroll
      for (int v = 0; v < E / 4; ++v) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p0 + 4 * v < hi) x = *reinterpret_cast<const float4*>(src + p0 + 4 * v);
        raw[4 * v] = __float_as_uint(x.x);
        raw[4 * v + 1] = __float_as_uint(x.y);
        raw[4 * v + 2] = __float_as_uint(x.z);
        raw[4 * v + 3] = __float_as_uint(x.w);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) raw[e] = (p0 + e < hi) ? __float_as_uint(src[p0 + e]) : 0u;
    }
    vmask = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ok = p0 + e >= lo && p0 + e < hi;
      vmask |= ok ? (1u << e) : 0u;
      key[e] = order_key(raw[e]);
    }
  };
  // runs f(c0) for every chunk with raw/key/vmask holding that chunk
  auto sweep = [&](auto f) {
    for (int c = 0; c < nchunks; ++c) {
      const int c0 = base + c * kChunk;
      if (!RESIDENT) load(c0);
      f(c0);
    }
  };

  // ---- 1. min / max of the finite valid scores -----------------------------
  if (RESIDENT) load(base);
  float vmin = INFINITY, vmax = -INFINITY;
  sweep([&](int) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ok = ((vmask >> e) & 1u) && finite_bits(raw[e]);
      const float x = __uint_as_float(raw[e]);
      vmin = fminf(vmin, ok ? x : INFINITY);
      vmax = fmaxf(vmax, ok ? x : -INFINITY);
    }
  });
  clear_words<NT>(sm.hist[0], kBins);
  if (tid == 0) sm.cnt = 0;
  block_min_max<NT>(vmin, vmax, sm.red);
  const LinBins lb = make_lin_bins(vmin, vmax);

  // ---- 2. threshold key ---------------------------------------------------
  sweep([&](int) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      atomicAdd(&sm.hist[0][lin_bin(raw[e], lb)], (vmask >> e) & 1u);
  });
  __syncthreads();
  const Bucket bk = block_find_bucket<true>(sm.hist[0], kBins, (uint32_t)k, sm.res);
  uint32_t kt, take;
  if (bk.count <= (uint32_t)kTopkListCap) {
    sweep([&](int) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (((vmask >> e) & 1u) && lin_bin(raw[e], lb) == bk.bin) {
          const uint32_t slot = atomicAdd(&sm.cnt, 1u);
          sm.list[slot] = key[e];   // slot < count <= the list capacity
        }
      }
    });
    __syncthreads();
    list_threshold<NT>(sm.list, (int)bk.count, bk.need, sm.res);
    kt = sm.res[0];
    take = sm.res[1];
  } else {
    uint32_t n_kt;
    radix_threshold<NT>(sm.hist, sm.res, (uint32_t)k, [&](auto f) {
      sweep([&](int) {
#pragma unroll
        for (int e = 0; e < E; ++e) f(key[e], ((vmask >> e) & 1u) != 0u);
      });
    }, &kt, &take, &n_kt);
  }

  // ---- 3. stable compaction in position order -----------------------------
  uint32_t run_gt = 0, run_eq = 0;
  int chunk = 0;
  sweep([&](int c0) {
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ok = (vmask >> e) & 1u;
      gt += (ok && key[e] > kt) ? 1u : 0u;
      eq += (ok && key[e] == kt) ? 1u : 0u;
    }
    uint32_t total;   // packed counts: a chunk holds <= 16K elements < 2^16
    const uint32_t excl = block_scan_excl<NT>(gt | (eq << 16), sm.scan[chunk & 1], total);
    uint32_t g_before = run_gt + (excl & 0xffffu);
    uint32_t e_before = run_eq + (excl >> 16);
    const int l0 = c0 + tid * E;
    int gq = l0 / I, gm = l0 - (l0 / I) * I;   // l = gq * I + gm, walked without division
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ok = (vmask >> e) & 1u;
      const bool is_gt = ok && key[e] > kt;
      const bool is_eq = ok && key[e] == kt;
      const uint32_t pos = g_before + (e_before < take ? e_before : take);
      if ((is_gt || (is_eq && e_before < take)) && pos < (uint32_t)k) {
        sm.out[pos] = make_float2(__uint_as_float(raw[e]), (float)((gq * S + r) * I + gm));
        sm.idx[pos] = l0 + e;
      }
      g_before += is_gt ? 1u : 0u;
      e_before += is_eq ? 1u : 0u;
      if (++gm == I) { gm = 0; ++gq; }
    }
    run_gt += total & 0xffffu;
    run_eq += total >> 16;
    ++chunk;
  });
  __syncthreads();

  // ---- 4. coalesced write-out (exactly k selections) ----------------------
  if (ocand) {
    if (out_vec) {
      for (int i = tid; i < k / 2; i += NT)
        reinterpret_cast<float4*>(ocand)[i] = reinterpret_cast<const float4*>(sm.out)[i];
    } else {
      for (int i = tid; i < k; i += NT) ocand[i] = sm.out[i];
    }
  }
  if (oidx) {
    for (int i = tid; i < k; i += NT) oidx[i] = sm.idx[i];
  }
}

template <int E>
__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(
    const float* __restrict__ logits, int64_t ld, int64_t shard_stride, int rows, int ctx,
    const int* __restrict__ row_starts, const int* __restrict__ row_ends, int k, int S, int I,
    int shard_first, int* __restrict__ local_idx, float* __restrict__ cand, int vec4,
    int cand_vec) {
  __shared__ TopkSmem sm;
  constexpr int NT = kTopkThreads;
  const int row = blockIdx.x;
  const int j = blockIdx.y;
  const int r = shard_first + j;
  const int tid = threadIdx.x;
  const float* src = logits + (int64_t)j * shard_stride + (int64_t)row * ld;

  // A shard row that fits one chunk is requested whole, from local position
  // 0, before its bounds are known, so that the bounds and the logits arrive
  // in one memory round trip; [lo, hi) then only masks.  16-byte loads stay
  // inside the row: ld is a multiple of 4 and at least the local length.  An
  // empty shard row reads nothing (ld may then be 0).
  constexpr int kChunk = NT * E;
  const int L = local_count(ctx, r, S, I);
  const bool whole = vec4 && L > 0 && L <= kChunk;
  uint32_t pre[E];
  if (whole) {
    const int p0 = tid * E;
#pragma unroll
    for (int v = 0; v < E / 4; ++v) {
      // positions past L (masked below) read position 0 instead: no branch
      const int pp = p0 + 4 * v < L ? p0 + 4 * v : 0;
      const float4 x = *reinterpret_cast<const float4*>(src + pp);
      pre[4 * v] = __float_as_uint(x.x);
      pre[4 * v + 1] = __float_as_uint(x.y);
      pre[4 * v + 2] = __float_as_uint(x.z);
      pre[4 * v + 3] = __float_as_uint(x.w);
    }
  }

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

  if (n <= k) {  // everything valid is selected
    for (int i = tid; i < k; i += NT) {
      int l = -1;
      float2 c = make_float2(-INFINITY, -1.0f);
      if (i < n) {
        l = lo + i;
        c = make_float2(src[l], (float)global_of(r, l, S, I));
      }
      if (oidx) oidx[i] = l;
      if (ocand) ocand[i] = c;
    }
    return;
  }
  if (whole) {
    topk_row<E, true>(sm, src, lo, hi, true, k, S, I, r, oidx, ocand, cand_vec != 0, pre);
    return;
  }
  // 16-byte loads start at the aligned position at or below lo; when that
  // would push a row that fits one chunk past it, the row is loaded
  // element-wise instead
  const bool vec = vec4 && (hi - (lo & ~3) <= kChunk || n > kChunk);
  const int span = hi - (vec ? (lo & ~3) : lo);
  if (span <= kChunk)
    topk_row<E, true>(sm, src, lo, hi, vec, k, S, I, r, oidx, ocand, cand_vec != 0, nullptr);
  else
    topk_row<E, false>(sm, src, lo, hi, vec, k, S, I, r, oidx, ocand, cand_vec != 0, nullptr);
}

int launch_topk_select(const float* logits, int64_t ld, int64_t shard_stride, int rows, int ctx,
                       const int* row_starts, const int* row_ends, int k, int S, int I,
                       int shard_first, int shard_count, int* local_idx, float* cand,
                       hipStream_t stream) {
  const int max_local = local_count(ctx, shard_first, S, I);
  const int vec4 =
      ((uintptr_t)logits % 16 == 0) && (ld % 4 == 0) && (shard_stride % 4 == 0) ? 1 : 0;
  const int cand_vec = ((uintptr_t)cand % 16 == 0) ? 1 : 0;   // k is even
  dim3 grid(rows, shard_count);
  // rows of up to 8K local positions are held 8 per thread, longer ones 16
  // per thread (swept in 16K chunks beyond 16K)
  if (max_local <= kTopkThreads * 8)
    hipLaunchKernelGGL((topk_select_kernel<8>), grid, dim3(kTopkThreads), 0, stream, logits, ld,
                       shard_stride, rows, ctx, row_starts, row_ends, k, S, I, shard_first,
                       local_idx, cand, vec4, cand_vec);
  else
    hipLaunchKernelGGL((topk_select_kernel<16>), grid, dim3(kTopkThreads), 0, stream, logits,
                       ld, shard_stride, rows, ctx, row_starts, row_ends, k, S, I, shard_first,
                       local_idx, cand, vec4, cand_vec);
  return 0;
}

}  // namespace dsa
