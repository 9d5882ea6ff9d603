// Global token ids -> per-shard physical cache slots, valid slots compacted
// to the front.
//
// What is computed (PR #46076 report, 实现拆解 item 4,
// `_convert_req_index_to_global_index_kernel` with DCP_SIZE / DCP_RANK /
// DCP_INTERLEAVE and its COMPACT_TO_FRONT branch): each shard keeps the ids
// it owns, de-interleaves each one to its local position, maps the position
// through its block table (slot = block * block_size + offset) and packs the
// slots at the front, -1 after them.
//
// How: one workgroup of 256 threads per (row, shard).  Thread t owns the E =
// k/256 contiguous ids [t*E, t*E+E) of the row (every shard's group reads the
// same ids, from L2 after the first); it resolves the ones its shard owns,
// a block exclusive scan of the per-thread counts (DPP inside each wave, one
// barrier across waves) gives every kept slot its position, so compaction
// keeps input order deterministically (no atomic slot counter).
#include "launchers.h"
#include "select_common.h"

namespace dsa {

constexpr int kConvThreads = 256;

template <int E>
__global__ __launch_bounds__(kConvThreads) void convert_index_kernel(
    const int* __restrict__ ids, int rows, int k, const int* __restrict__ row_req,
    int num_reqs, const int* __restrict__ block_table, int64_t bt_ld, int64_t bt_stride,
    int bs, int S, int I, int first, int* __restrict__ slots, int* __restrict__ counts,
    int vec) {
  constexpr int NT = kConvThreads;
  __shared__ uint32_t s_scan[NT / kWave];

  const int row = blockIdx.x;
  const int j = blockIdx.y;
  const int r = first + j;
  const int tid = threadIdx.x;
  const int req = row_req ? row_req[row] : row;
  const bool req_ok = req >= 0 && req < num_reqs;
  const int* my_ids = ids + (int64_t)row * k + tid * E;
  const int* bt = block_table + (int64_t)j * bt_stride + (int64_t)(req_ok ? req : 0) * bt_ld;
  int* dst = slots + ((int64_t)j * rows + row) * k;

  int g[E];
  if (vec) {
#pragma unroll
    for (int v = 0; v < E; v += 2) {
      const int2 x = *reinterpret_cast<const int2*>(my_ids + v);
      g[v] = x.x;
      g[v + 1] = x.y;
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) g[e] = my_ids[e];
  }

  // local position -> block-table column for the ids this shard keeps
  int col[E], off[E];
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    col[e] = -1;
    off[e] = 0;
    if (req_ok && g[e] >= 0 && owner_of(g[e], S, I) == r) {
      const int l = local_of(g[e], S, I);
      const int c = l / bs;
      if ((int64_t)c < bt_ld) {
        col[e] = c;
        off[e] = l - c * bs;
        ++cnt;
      }
    }
  }
  int blk[E];
#pragma unroll
  for (int e = 0; e < E; ++e) blk[e] = col[e] >= 0 ? bt[col[e]] : 0;

  uint32_t total;
  uint32_t pos = block_scan_excl<NT>(cnt, s_scan, total);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (col[e] >= 0) dst[pos++] = blk[e] * bs + off[e];
  }
  for (int i = (int)total + tid; i < k; i += NT) dst[i] = -1;
  if (tid == 0 && counts) counts[(int64_t)j * rows + row] = (int)total;
}

int launch_convert_index(const int* ids, int rows, int k, const int* row_req, int num_reqs,
                         const int* block_table, int64_t bt_ld, int64_t bt_stride, int bs,
                         int S, int I, int first, int count, int* slots, int* counts,
                         hipStream_t stream) {
  const int vec = ((uintptr_t)ids % 8 == 0) ? 1 : 0;
  dim3 grid(rows, count);
#define DSA_CONVERT(E)                                                                          \
  hipLaunchKernelGGL((convert_index_kernel<E>), grid, dim3(kConvThreads), 0, stream, ids, rows, \
                     k, row_req, num_reqs, block_table, bt_ld, bt_stride, bs, S, I, first,      \
                     slots, counts, vec)
  switch (k / kConvThreads) {   // k is 512, 1024 or 2048
    case 2: DSA_CONVERT(2); break;
    case 4: DSA_CONVERT(4); break;
    default: DSA_CONVERT(8); break;
  }
#undef DSA_CONVERT
  return 0;
}

}  // namespace dsa
