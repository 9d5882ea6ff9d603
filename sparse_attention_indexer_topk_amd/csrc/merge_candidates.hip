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
//
// merge_convert_kernel continues in the same workgroup with the index
// conversion (PR #46076 report, 实现拆解 item 4; the same result as
// convert_index on the merged ids): the merged ids are already in LDS in
// ascending order, so the per-shard compaction needs neither a second launch
// nor a reload of the ids.  The merge of a row is latency-bound and occupies
// one CU, so when rows alone leave CUs idle each (row, shard group) gets its
// own workgroup, up to one per CU: it repeats the row's merge (its
// candidates come from L2: the row's workgroups are launched on one XCD) and
// converts only its group's shards; the conversion's stores are then spread
// over more CUs.
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
  uint32_t scan[2][kMergeThreads / kWave];   // two, for back-to-back scans
  uint32_t res[4];
  uint32_t cnt;
  uint32_t nvalid;
};

// order key -> fp32 bits; exact except that -0 comes back as +0 and every
// NaN as one NaN, neither of which changes a bin or a comparison
__device__ __forceinline__ uint32_t key_to_bits(uint32_t key) {
  return (key & 0x80000000u) ? (key ^ 0x80000000u) : ~key;
}

// Returns the number of ids kept; they are left in sm.stage in ascending
// order (every thread has passed the barrier after they were written).
template <int E, bool RESIDENT>
__device__ __forceinline__ int merge_row(MergeSmem& sm, const float* __restrict__ src,
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
    uint32_t pos = written + block_scan_excl<NT>(cnt, sm.scan[0], total);
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
  if (out)
    for (int i = tid; i < k; i += NT) out[i] = i < n_out ? sm.stage[i] : -1;
  return n_out;
}

// ---- index conversion of the merged ids (merge_convert_kernel) -------------
struct ConvertArgs {
  const int* row_req;       // nullable: row i -> request i
  int num_reqs;
  const int* block_table;   // [count][num_reqs][bt_ld], slice j at + j * bt_stride
  int64_t bt_ld, bt_stride;
  int bs, S, I, first, count, rows;
  int* slots;               // [count][rows][k]
  int* counts;              // nullable, [count][rows]
  int groups;               // workgroups per row, each converting `per` shards
  int per;
};

// Thread t resolves merged positions [t*P, t*P + P): owner shard, local
// position, block-table slot (all lookups in flight together).  Per shard,
// a block exclusive scan of the per-thread counts places the slots in input
// order; two shards share one scan as 16-bit fields (a row keeps at most 2048
// ids, so no field carries into the next).
__device__ __forceinline__ void convert_tail(MergeSmem& sm, int n_out, int k, int row,
                                             int j_lo, int j_hi, const ConvertArgs& cv) {
  constexpr int NT = kMergeThreads;
  constexpr int P = kMergeMaxK / NT;
  const int tid = threadIdx.x;
  const int req = cv.row_req ? cv.row_req[row] : row;
  const bool req_ok = req >= 0 && req < cv.num_reqs;
  int jj[P], slot[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    jj[p] = -1;
    slot[p] = 0;
    const int i = tid * P + p;
    if (req_ok && i < n_out) {
      const int g = sm.stage[i];
      const int j = owner_of(g, cv.S, cv.I) - cv.first;
      if (j >= j_lo && j < j_hi) {
        const int l = local_of(g, cv.S, cv.I);
        const int c = l / cv.bs;
        if ((int64_t)c < cv.bt_ld) {
          jj[p] = j;
          slot[p] = cv.block_table[(int64_t)j * cv.bt_stride + (int64_t)req * cv.bt_ld + c] *
                        cv.bs + (l - c * cv.bs);
        }
      }
    }
  }
  for (int j0 = j_lo; j0 < j_hi; j0 += 2) {
    uint32_t c = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) c += jj[p] == j0 ? 1u : (jj[p] == j0 + 1 ? 0x10000u : 0u);
    uint32_t total;
    const uint32_t pos = block_scan_excl<NT>(c, sm.scan[((j0 - j_lo) >> 1) & 1], total);
    for (int h = 0; h < 2 && j0 + h < j_hi; ++h) {
      const int j = j0 + h;
      uint32_t ps = (pos >> (16 * h)) & 0xffffu;
      const int tot = (int)((total >> (16 * h)) & 0xffffu);
      int* dst = cv.slots + ((int64_t)j * cv.rows + row) * k;
#pragma unroll
      for (int p = 0; p < P; ++p)
        if (jj[p] == j) dst[ps++] = slot[p];
      for (int i = tot + tid; i < k; i += NT) dst[i] = -1;
      if (tid == 0 && cv.counts) cv.counts[(int64_t)j * cv.rows + row] = tot;
    }
  }
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

template <int E>
__global__ __launch_bounds__(kMergeThreads) void merge_convert_kernel(
    const float* __restrict__ cand, int n_cand, int k, int id_bound, int* __restrict__ ids,
    int vec, ConvertArgs cv) {
  __shared__ MergeSmem sm;
  // XCD-aware order: launch index L -> (row, group) with the G groups of a
  // row 8 launch indices apart inside a run of 8*G (same XCD, same round)
  const int G = cv.groups;
  const int L = blockIdx.x;
  const int b = L / (8 * G), w = L % (8 * G);
  const int nr = cv.rows - 8 * b < 8 ? cv.rows - 8 * b : 8;
  const int row = 8 * b + w % nr;
  const int grp = w / nr;
  const int j_lo = grp * cv.per;
  const int j_hi = j_lo + cv.per < cv.count ? j_lo + cv.per : cv.count;
  const float* src = cand + (int64_t)row * n_cand * 2;
  int* out = (ids && grp == 0) ? ids + (int64_t)row * k : nullptr;
  const int n_out = n_cand <= kMergeThreads * E
                        ? merge_row<E, true>(sm, src, n_cand, k, id_bound, vec != 0, out)
                        : merge_row<E, false>(sm, src, n_cand, k, id_bound, vec != 0, out);
  convert_tail(sm, n_out, k, row, j_lo, j_hi, cv);
}

int launch_merge_convert(const float* cand, int rows, int n_cand, int k, int id_bound, int* ids,
                         const int* row_req, int num_reqs, const int* block_table, int64_t bt_ld,
                         int64_t bt_stride, int bs, int S, int I, int first, int count,
                         int* slots, int* counts, hipStream_t stream) {
  const int vec = ((uintptr_t)cand % 16 == 0 && n_cand % 2 == 0) ? 1 : 0;
  // as many shard groups per row as keep the launch within one workgroup
  // per CU (a second merge on a CU costs more than the conversion it
  // spreads); with 256 rows or more, one workgroup per row converts every
  // shard
  constexpr int kCUs = 256;
  const int g0 = std::max(1, std::min(count, kCUs / std::max(rows, 1)));
  const int per = (count + g0 - 1) / g0;
  const int groups = (count + per - 1) / per;   // no empty group
  const ConvertArgs cv{row_req, num_reqs, block_table, bt_ld, bt_stride, bs, S, I, first,
                       count, rows, slots, counts, groups, per};
  const dim3 grid((unsigned)((int64_t)rows * groups));
  if (n_cand <= kMergeThreads * 8)
    hipLaunchKernelGGL((merge_convert_kernel<8>), grid, dim3(kMergeThreads), 0, stream, cand,
                       n_cand, k, id_bound, ids, vec, cv);
  else
    hipLaunchKernelGGL((merge_convert_kernel<16>), grid, dim3(kMergeThreads), 0, stream, cand,
                       n_cand, k, id_bound, ids, vec, cv);
  return 0;
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
