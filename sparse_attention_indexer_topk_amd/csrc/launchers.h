// Internal launchers: argument checking happens in api.hip before these run.
#pragma once

#include "dsa_common.h"

namespace dsa {

int launch_topk_select(const float* logits, int64_t ld, int64_t shard_stride, int rows, int ctx,
                       const int* row_starts, const int* row_ends, int k, int S, int I,
                       int shard_first, int shard_count, int* local_idx, float* cand,
                       hipStream_t stream);

int launch_merge_candidates(const float* cand, int rows, int n_cand, int k, int id_bound,
                            int* ids, hipStream_t stream);

int launch_merge_convert(const float* cand, int rows, int n_cand, int k, int id_bound, int* ids,
                         const int* row_req, int num_reqs, const int* block_table, int64_t bt_ld,
                         int64_t bt_stride, int bs, int S, int I, int first, int count,
                         int* slots, int* counts, hipStream_t stream);

int launch_convert_index(const int* ids, int rows, int k, const int* row_req, int num_reqs,
                         const int* block_table, int64_t bt_ld, int64_t bt_stride, int bs,
                         int S, int I, int first, int count, int* slots, int* counts,
                         hipStream_t stream);

int launch_sparse_mla_decode(const void* q, int rows, int heads, const void* cache, bool fp8,
                             const float* cache_scale, int64_t num_slots, const int* slots,
                             const int* counts, int k, int n_parts, int splits, float sm_scale,
                             void* out, bool f32out, float* lse, hipStream_t stream);

int launch_lse_combine(const void* part_out, bool f32in, const float* part_lse, int P, int rows,
                       int heads, int dim, void* out, float* lse_out, hipStream_t stream);

int launch_cache_insert(const void* kv_c, int64_t kv_ld, const void* k_pe, int64_t pe_ld, int T,
                        void* cache, int cache_kind, const float* cache_scale,
                        const int64_t* slot_mapping, int64_t num_slots, hipStream_t stream);

// Indexer-key branch of the fused norm + RoPE launch (fields unused when the
// branch does not run).
struct IndexerArgs {
  const uint16_t* k;     // [T][ld] bf16, first 128 used
  int64_t ld;
  const uint16_t* w;     // [128] bf16
  float eps;
  uint16_t* out;         // [T][128] bf16 (nullable)
  uint8_t* cache;        // [num_slots][128] e4m3 (nullable)
  const float* scale;    // device scalar (with cache)
  int64_t num_slots;
};

int launch_fused_rmsnorm_rope(const void* kv_c, int64_t kv_ld, const void* k_pe, int64_t pe_ld,
                              int T, const void* w, float eps, const float* cos_sin, int n_pos,
                              const int* positions, void* kv_out, void* pe_out, void* cache,
                              int cache_kind, const float* cache_scale,
                              const int64_t* slot_mapping, int64_t num_slots, bool latent,
                              const IndexerArgs& ix, bool indexer, hipStream_t stream);

int launch_floor(int workgroups, int threads, hipStream_t stream);

}  // namespace dsa
