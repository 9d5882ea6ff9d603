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
// How: one workgroup per row handles every shard of the run.  Ids are read
// 256 at a time; for each shard a wave ballot marks the lanes whose id the
// shard owns, the lane's rank among them is a popcount of the lower lanes,
// and per-wave totals give the block offsets.  The compaction therefore keeps
// input order deterministically (no atomic slot counter).
#include "launchers.h"

namespace dsa {

constexpr int kConvThreads = 256;

__global__ __launch_bounds__(kConvThreads) void convert_index_kernel(
    const int* __restrict__ ids, int rows, int k, const int* __restrict__ row_req,
    int num_reqs, const int* __restrict__ block_table, int64_t bt_ld, int64_t bt_stride,
    int bs, int S, int I, int first, int count, int* __restrict__ slots,
    int* __restrict__ counts) {
  constexpr int NT = kConvThreads;
  constexpr int NW = NT / kWave;
  __shared__ uint32_t s_wave[16][NW];
  __shared__ uint32_t s_run[16];

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int req = row_req ? row_req[row] : row;
  const bool req_ok = req >= 0 && req < num_reqs;
  const int* my_ids = ids + (int64_t)row * k;

  if (tid < count) s_run[tid] = 0;
  __syncthreads();

  for (int base = 0; base < k; base += NT) {
    const int i = base + tid;
    const int g = (i < k && req_ok) ? my_ids[i] : -1;
    int sh = -1, slot = -1;
    if (g >= 0) {
      const int r = owner_of(g, S, I);
      if (r >= first && r < first + count) {
        const int l = local_of(g, S, I);
        const int col = l / bs;
        if ((int64_t)col < bt_ld) {
          const int blk = block_table[(int64_t)(r - first) * bt_stride + (int64_t)req * bt_ld + col];
          slot = blk * bs + l % bs;
          sh = r - first;
        }
      }
    }
    uint32_t my_rank = 0;
    for (int s = 0; s < count; ++s) {
      const uint64_t m = __ballot(sh == s);
      if (lane == 0) s_wave[s][wave] = (uint32_t)__popcll(m);
      if (sh == s) my_rank = (uint32_t)__popcll(m & lt_mask);
    }
    __syncthreads();
    if (sh >= 0) {
      uint32_t pos = s_run[sh] + my_rank;
      for (int w = 0; w < wave; ++w) pos += s_wave[sh][w];
      if (pos < (uint32_t)k) slots[((int64_t)sh * rows + row) * k + pos] = slot;
    }
    __syncthreads();
    if (tid < count) {
      uint32_t add = 0;
      for (int w = 0; w < NW; ++w) add += s_wave[tid][w];
      s_run[tid] += add;
    }
    __syncthreads();
  }

  for (int s = 0; s < count; ++s) {
    const uint32_t c = s_run[s];
    int* dst = slots + ((int64_t)s * rows + row) * k;
    for (int i = (int)c + tid; i < k; i += NT) dst[i] = -1;
    if (tid == 0 && counts) counts[(int64_t)s * rows + row] = (int)c;
  }
}

int launch_convert_index(const int* ids, int rows, int k, const int* row_req, int num_reqs,
                         const int* block_table, int64_t bt_ld, int64_t bt_stride, int bs,
                         int S, int I, int first, int count, int* slots, int* counts,
                         hipStream_t stream) {
  hipLaunchKernelGGL(convert_index_kernel, dim3(rows), dim3(kConvThreads), 0, stream, ids,
                     rows, k, row_req, num_reqs, block_table, bt_ld, bt_stride, bs, S, I,
                     first, count, slots, counts);
  return 0;
}

}  // namespace dsa
