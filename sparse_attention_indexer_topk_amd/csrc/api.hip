// C ABI of the DSA library: host-side argument validation, then a launch on
// the caller's stream.  Nothing here touches HIP before validation passes.
#include <stdarg.h>
#include <stdio.h>

#include "dsa.h"
#include "launchers.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, uintptr_t a) { return p == nullptr || ((uintptr_t)p % a) == 0; }
bool k_ok(int32_t k) { return k == 512 || k == 1024 || k == 2048; }

int check_shards(const char* fn, int32_t S, int32_t I, int32_t first, int32_t count) {
  if (S < 1 || S > DSA_MAX_SHARDS)
    return fail(DSA_ERR_INVALID_ARG, "%s: num_shards=%d outside [1, %d]", fn, S, DSA_MAX_SHARDS);
  if (I < 1 || (int64_t)I * S > DSA_MAX_ID)
    return fail(DSA_ERR_INVALID_ARG, "%s: interleave=%d invalid for %d shards", fn, I, S);
  if (first < 0 || count < 1 || first + count > S)
    return fail(DSA_ERR_INVALID_ARG, "%s: shard range [%d, %d) outside [0, %d)", fn, first,
                first + count, S);
  return DSA_OK;
}

int launched(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_last_error(void) { return g_err; }

int dsa_version(void) { return 100; }

int dsa_topk_select(const float* logits, int64_t ld, int64_t shard_stride, int32_t rows,
                    int32_t ctx, const int32_t* row_starts, const int32_t* row_ends, int32_t k,
                    int32_t num_shards, int32_t interleave, int32_t shard_first,
                    int32_t shard_count, int32_t* local_idx, float* cand, hipStream_t stream) {
  const char* fn = "dsa_topk_select";
  if (!logits) return fail(DSA_ERR_INVALID_ARG, "%s: logits is NULL", fn);
  if (!local_idx && !cand) return fail(DSA_ERR_INVALID_ARG, "%s: no output given", fn);
  if (rows < 0) return fail(DSA_ERR_INVALID_ARG, "%s: rows=%d < 0", fn, rows);
  if (!k_ok(k)) return fail(DSA_ERR_UNSUPPORTED_K, "%s: k=%d not in {512, 1024, 2048}", fn, k);
  if (int rc = check_shards(fn, num_shards, interleave, shard_first, shard_count)) return rc;
  if (ctx < 0 || ctx > DSA_MAX_ID)
    return fail(DSA_ERR_INVALID_ARG, "%s: ctx=%d outside [0, 2^24]", fn, ctx);
  const int need_ld = dsa::local_count(ctx, shard_first, num_shards, interleave);
  if (ld < need_ld)
    return fail(DSA_ERR_INVALID_ARG, "%s: ld=%lld < %d local positions of shard %d", fn,
                (long long)ld, need_ld, shard_first);
  if (shard_stride < 0 || (shard_count > 1 && shard_stride < (int64_t)rows * ld))
    return fail(DSA_ERR_INVALID_ARG, "%s: shard_stride=%lld overlaps slices", fn,
                (long long)shard_stride);
  if (!aligned(logits, 4) || !aligned(local_idx, 4) || !aligned(cand, 8))
    return fail(DSA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  if (rows == 0) return DSA_OK;
  dsa::launch_topk_select(logits, ld, shard_stride, rows, ctx, row_starts, row_ends, k,
                          num_shards, interleave, shard_first, shard_count, local_idx, cand,
                          stream);
  return launched(fn);
}

int dsa_merge_candidates(const float* cand, int32_t rows, int32_t n_cand, int32_t k,
                         int32_t id_bound, int32_t* ids, hipStream_t stream) {
  const char* fn = "dsa_merge_candidates";
  if (!cand || !ids) return fail(DSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (rows < 0) return fail(DSA_ERR_INVALID_ARG, "%s: rows=%d < 0", fn, rows);
  if (!k_ok(k)) return fail(DSA_ERR_UNSUPPORTED_K, "%s: k=%d not in {512, 1024, 2048}", fn, k);
  if (n_cand < 1 || n_cand > DSA_MAX_SHARDS * k)
    return fail(DSA_ERR_INVALID_ARG, "%s: n_cand=%d outside [1, 16*k]", fn, n_cand);
  if (id_bound < 1 || id_bound > DSA_MAX_ID)
    return fail(DSA_ERR_INVALID_ARG, "%s: id_bound=%d outside [1, 2^24]", fn, id_bound);
  if (!aligned(cand, 8) || !aligned(ids, 4))
    return fail(DSA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  if (rows == 0) return DSA_OK;
  dsa::launch_merge_candidates(cand, rows, n_cand, k, id_bound, ids, stream);
  return launched(fn);
}

int dsa_convert_index(const int32_t* ids, int32_t rows, int32_t k, const int32_t* row_req,
                      int32_t num_reqs, const int32_t* block_table, int64_t bt_ld,
                      int64_t bt_shard_stride, int32_t block_size, int32_t num_shards,
                      int32_t interleave, int32_t shard_first, int32_t shard_count,
                      int32_t* slots, int32_t* counts, hipStream_t stream) {
  const char* fn = "dsa_convert_index";
  if (!ids || !block_table || !slots) return fail(DSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (rows < 0) return fail(DSA_ERR_INVALID_ARG, "%s: rows=%d < 0", fn, rows);
  if (!k_ok(k)) return fail(DSA_ERR_UNSUPPORTED_K, "%s: k=%d not in {512, 1024, 2048}", fn, k);
  if (int rc = check_shards(fn, num_shards, interleave, shard_first, shard_count)) return rc;
  if (num_reqs < 1) return fail(DSA_ERR_INVALID_ARG, "%s: num_reqs=%d < 1", fn, num_reqs);
  if (bt_ld < 1) return fail(DSA_ERR_INVALID_ARG, "%s: bt_ld=%lld < 1", fn, (long long)bt_ld);
  if (bt_shard_stride < 0 || (shard_count > 1 && bt_shard_stride < (int64_t)num_reqs * bt_ld))
    return fail(DSA_ERR_INVALID_ARG, "%s: bt_shard_stride=%lld overlaps slices", fn,
                (long long)bt_shard_stride);
  if (block_size < 1) return fail(DSA_ERR_INVALID_ARG, "%s: block_size=%d < 1", fn, block_size);
  if (rows == 0) return DSA_OK;
  dsa::launch_convert_index(ids, rows, k, row_req, num_reqs, block_table, bt_ld, bt_shard_stride,
                            block_size, num_shards, interleave, shard_first, shard_count, slots,
                            counts, stream);
  return launched(fn);
}

int dsa_merge_convert(const float* cand, int32_t rows, int32_t n_cand, int32_t k,
                      int32_t id_bound, int32_t* ids, const int32_t* row_req, int32_t num_reqs,
                      const int32_t* block_table, int64_t bt_ld, int64_t bt_shard_stride,
                      int32_t block_size, int32_t num_shards, int32_t interleave,
                      int32_t shard_first, int32_t shard_count, int32_t* slots,
                      int32_t* counts, hipStream_t stream) {
  const char* fn = "dsa_merge_convert";
  if (!cand || !block_table || !slots) return fail(DSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (rows < 0) return fail(DSA_ERR_INVALID_ARG, "%s: rows=%d < 0", fn, rows);
  if (!k_ok(k)) return fail(DSA_ERR_UNSUPPORTED_K, "%s: k=%d not in {512, 1024, 2048}", fn, k);
  if (n_cand < 1 || n_cand > DSA_MAX_SHARDS * k)
    return fail(DSA_ERR_INVALID_ARG, "%s: n_cand=%d outside [1, 16*k]", fn, n_cand);
  if (id_bound < 1 || id_bound > DSA_MAX_ID)
    return fail(DSA_ERR_INVALID_ARG, "%s: id_bound=%d outside [1, 2^24]", fn, id_bound);
  if (int rc = check_shards(fn, num_shards, interleave, shard_first, shard_count)) return rc;
  if (num_reqs < 1) return fail(DSA_ERR_INVALID_ARG, "%s: num_reqs=%d < 1", fn, num_reqs);
  if (bt_ld < 1) return fail(DSA_ERR_INVALID_ARG, "%s: bt_ld=%lld < 1", fn, (long long)bt_ld);
  if (bt_shard_stride < 0 || (shard_count > 1 && bt_shard_stride < (int64_t)num_reqs * bt_ld))
    return fail(DSA_ERR_INVALID_ARG, "%s: bt_shard_stride=%lld overlaps slices", fn,
                (long long)bt_shard_stride);
  if (block_size < 1) return fail(DSA_ERR_INVALID_ARG, "%s: block_size=%d < 1", fn, block_size);
  if (!aligned(cand, 8) || !aligned(ids, 4))
    return fail(DSA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  if (rows == 0) return DSA_OK;
  dsa::launch_merge_convert(cand, rows, n_cand, k, id_bound, ids, row_req, num_reqs, block_table,
                            bt_ld, bt_shard_stride, block_size, num_shards, interleave,
                            shard_first, shard_count, slots, counts, stream);
  return launched(fn);
}

int dsa_sparse_mla_decode(const void* q, int32_t rows, int32_t heads, const void* cache,
                          int32_t cache_dtype, const float* cache_scale, int64_t num_slots,
                          const int32_t* slots, const int32_t* counts, int32_t k,
                          int32_t n_parts, int32_t splits, float sm_scale, void* out,
                          int32_t out_dtype, float* lse, hipStream_t stream) {
  const char* fn = "dsa_sparse_mla_decode";
  if (out_dtype != DSA_BF16 && out_dtype != DSA_FP32)
    return fail(DSA_ERR_UNSUPPORTED_DTYPE, "%s: output dtype %d is not bf16 or fp32", fn,
                out_dtype);
  if (!q || !cache || !slots || !out || !lse)
    return fail(DSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (rows < 0) return fail(DSA_ERR_INVALID_ARG, "%s: rows=%d < 0", fn, rows);
  if (heads < 16 || heads % 16 != 0)
    return fail(DSA_ERR_INVALID_ARG, "%s: heads=%d is not a positive multiple of 16", fn, heads);
  if (!k_ok(k)) return fail(DSA_ERR_UNSUPPORTED_K, "%s: k=%d not in {512, 1024, 2048}", fn, k);
  if (n_parts < 1 || n_parts > 65535)
    return fail(DSA_ERR_INVALID_ARG, "%s: n_parts=%d outside [1, 65535]", fn, n_parts);
  if (splits < 1 || splits > 64 || (int64_t)n_parts * splits > 65535)
    return fail(DSA_ERR_INVALID_ARG, "%s: splits=%d outside [1, 64] (or n_parts*splits > 65535)",
                fn, splits);
  if (cache_dtype != DSA_BF16 && cache_dtype != DSA_FP8_E4M3)
    return fail(DSA_ERR_UNSUPPORTED_DTYPE, "%s: cache dtype %d is not bf16 or fp8 e4m3", fn,
                cache_dtype);
  if (cache_dtype == DSA_FP8_E4M3 && !cache_scale)
    return fail(DSA_ERR_INVALID_ARG, "%s: fp8 cache needs cache_scale", fn);
  if (num_slots < 0) return fail(DSA_ERR_INVALID_ARG, "%s: num_slots < 0", fn);
  // the kernel numbers its workgroups (rows x parts x splits x head groups of
  // 128) with 32-bit integers
  if ((int64_t)rows * n_parts * splits * ((heads + 127) / 128) > 0x7fffffffLL)
    return fail(DSA_ERR_INVALID_ARG, "%s: rows x n_parts x splits x head groups exceeds 2^31 - 1",
                fn);
  if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(out, 16) || !aligned(slots, 4) ||
      !aligned(lse, 4) || !aligned(cache_scale, 4))
    return fail(DSA_ERR_INVALID_ARG, "%s: misaligned pointer (q, cache, out need 16 bytes)", fn);
  if (rows == 0) return DSA_OK;
  dsa::launch_sparse_mla_decode(q, rows, heads, cache, cache_dtype == DSA_FP8_E4M3, cache_scale,
                                num_slots, slots, counts, k, n_parts, splits, sm_scale, out,
                                out_dtype == DSA_FP32, lse, stream);
  return launched(fn);
}

int dsa_lse_combine(const void* part_out, int32_t part_dtype, const float* part_lse,
                    int32_t n_parts, int32_t rows, int32_t heads, int32_t dim, void* out,
                    float* lse_out, hipStream_t stream) {
  const char* fn = "dsa_lse_combine";
  if (part_dtype != DSA_BF16 && part_dtype != DSA_FP32)
    return fail(DSA_ERR_UNSUPPORTED_DTYPE, "%s: partial dtype %d is not bf16 or fp32", fn,
                part_dtype);
  if (!part_out || !part_lse || !out) return fail(DSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (n_parts < 1 || n_parts > 64)
    return fail(DSA_ERR_INVALID_ARG, "%s: n_parts=%d outside [1, 64]", fn, n_parts);
  if (rows < 0 || heads < 0) return fail(DSA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (dim < 8 || dim % 8 != 0)
    return fail(DSA_ERR_INVALID_ARG, "%s: dim=%d is not a positive multiple of 8", fn, dim);
  if (!aligned(part_out, 16) || !aligned(out, 16) || !aligned(part_lse, 4) || !aligned(lse_out, 4))
    return fail(DSA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  if (rows == 0 || heads == 0) return DSA_OK;
  dsa::launch_lse_combine(part_out, part_dtype == DSA_FP32, part_lse, n_parts, rows, heads, dim,
                          out, lse_out, stream);
  return launched(fn);
}

int dsa_fused_rmsnorm_rope(const void* kv_c, int64_t kv_c_ld, const void* k_pe, int64_t k_pe_ld,
                           int32_t T, const void* rms_w, float eps, const float* cos_sin,
                           int32_t n_pos, const int32_t* positions, void* kv_c_out,
                           void* k_pe_out, void* cache, int32_t cache_dtype,
                           const float* cache_scale, const int64_t* slot_mapping,
                           int64_t num_slots, const void* index_k, int64_t index_k_ld,
                           const void* index_w, float index_eps, void* index_k_out,
                           void* index_cache, const float* index_cache_scale,
                           int64_t index_num_slots, hipStream_t stream) {
  const char* fn = "dsa_fused_rmsnorm_rope";
  if (T < 0) return fail(DSA_ERR_INVALID_ARG, "%s: T=%d < 0", fn, T);
  // the early return of the profiling path: every output NULL and no slot
  // mapping, so nothing is materialised or inserted
  if (!kv_c_out && !k_pe_out && !index_k_out && !slot_mapping) return DSA_OK;
  if (slot_mapping && !cache && !index_cache)
    return fail(DSA_ERR_INVALID_ARG, "%s: slot_mapping without a cache", fn);
  const bool latent = kv_c_out || k_pe_out || (slot_mapping && cache);
  const bool indexer = index_k_out || (slot_mapping && index_cache);
  if (!cos_sin || !positions) return fail(DSA_ERR_INVALID_ARG, "%s: NULL cos_sin/positions", fn);
  if (n_pos < 1) return fail(DSA_ERR_INVALID_ARG, "%s: n_pos=%d < 1", fn, n_pos);
  int kind = 0;
  if (latent) {
    if (!kv_c || !k_pe || !rms_w) return fail(DSA_ERR_INVALID_ARG, "%s: NULL input pointer", fn);
    if (kv_c_ld < DSA_VALUE_DIM || kv_c_ld % 8 != 0)
      return fail(DSA_ERR_INVALID_ARG, "%s: kv_c_ld=%lld must be >= 512 and a multiple of 8", fn,
                  (long long)kv_c_ld);
    if (k_pe_ld < DSA_ROPE_DIM || k_pe_ld % 2 != 0)
      return fail(DSA_ERR_INVALID_ARG, "%s: k_pe_ld=%lld must be >= 64 and even", fn,
                  (long long)k_pe_ld);
    if (slot_mapping && cache) {
      if (cache_dtype == DSA_BF16) kind = 1;
      else if (cache_dtype == DSA_FP8_E4M3) kind = 2;
      else return fail(DSA_ERR_UNSUPPORTED_DTYPE, "%s: cache dtype %d is not bf16 or fp8", fn,
                       cache_dtype);
      if (kind == 2 && !cache_scale)
        return fail(DSA_ERR_INVALID_ARG, "%s: fp8 cache needs cache_scale", fn);
      if (num_slots < 0) return fail(DSA_ERR_INVALID_ARG, "%s: num_slots < 0", fn);
    }
  }
  if (indexer) {
    if (!index_k || !index_w)
      return fail(DSA_ERR_INVALID_ARG, "%s: NULL index_k/index_w", fn);
    if (index_k_ld < DSA_INDEX_DIM || index_k_ld % 2 != 0)
      return fail(DSA_ERR_INVALID_ARG, "%s: index_k_ld=%lld must be >= 128 and even", fn,
                  (long long)index_k_ld);
    if (slot_mapping && index_cache) {
      if (!index_cache_scale)
        return fail(DSA_ERR_INVALID_ARG, "%s: the fp8 indexer cache needs its scale", fn);
      if (index_num_slots < 0) return fail(DSA_ERR_INVALID_ARG, "%s: index_num_slots < 0", fn);
    }
  }
  if (!aligned(kv_c, 16) || !aligned(k_pe, 4) || !aligned(rms_w, 16) || !aligned(kv_c_out, 16) ||
      !aligned(k_pe_out, 4) || !aligned(cache, 16) || !aligned(cos_sin, 4) ||
      !aligned(positions, 4) || !aligned(slot_mapping, 8) || !aligned(index_k, 4) ||
      !aligned(index_w, 4) || !aligned(index_k_out, 4) || !aligned(index_cache, 2) ||
      !aligned(index_cache_scale, 4))
    return fail(DSA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  if (T == 0 || (!latent && !indexer)) return DSA_OK;
  dsa::IndexerArgs ix{};
  if (indexer) {
    ix.k = reinterpret_cast<const uint16_t*>(index_k);
    ix.ld = index_k_ld;
    ix.w = reinterpret_cast<const uint16_t*>(index_w);
    ix.eps = index_eps;
    ix.out = reinterpret_cast<uint16_t*>(index_k_out);
    ix.cache = slot_mapping ? reinterpret_cast<uint8_t*>(index_cache) : nullptr;
    ix.scale = index_cache_scale;
    ix.num_slots = index_num_slots;
  }
  dsa::launch_fused_rmsnorm_rope(kv_c, kv_c_ld, k_pe, k_pe_ld, T, rms_w, eps, cos_sin, n_pos,
                                 positions, kv_c_out, k_pe_out, cache, kind, cache_scale,
                                 slot_mapping, num_slots, latent, ix, indexer, stream);
  return launched(fn);
}

int dsa_cache_insert(const void* kv_c, int64_t kv_c_ld, const void* k_pe, int64_t k_pe_ld,
                     int32_t T, void* cache, int32_t cache_dtype, const float* cache_scale,
                     const int64_t* slot_mapping, int64_t num_slots, hipStream_t stream) {
  const char* fn = "dsa_cache_insert";
  if (T < 0) return fail(DSA_ERR_INVALID_ARG, "%s: T=%d < 0", fn, T);
  if (!kv_c || !k_pe || !cache || !slot_mapping)
    return fail(DSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (kv_c_ld < DSA_VALUE_DIM || kv_c_ld % 8 != 0)
    return fail(DSA_ERR_INVALID_ARG, "%s: kv_c_ld=%lld must be >= 512 and a multiple of 8", fn,
                (long long)kv_c_ld);
  if (k_pe_ld < DSA_ROPE_DIM || k_pe_ld % 2 != 0)
    return fail(DSA_ERR_INVALID_ARG, "%s: k_pe_ld=%lld must be >= 64 and even", fn,
                (long long)k_pe_ld);
  int kind;
  if (cache_dtype == DSA_BF16) kind = 1;
  else if (cache_dtype == DSA_FP8_E4M3) kind = 2;
  else return fail(DSA_ERR_UNSUPPORTED_DTYPE, "%s: cache dtype %d is not bf16 or fp8", fn,
                   cache_dtype);
  if (kind == 2 && !cache_scale) return fail(DSA_ERR_INVALID_ARG, "%s: fp8 cache needs cache_scale", fn);
  if (num_slots < 0) return fail(DSA_ERR_INVALID_ARG, "%s: num_slots < 0", fn);
  if (!aligned(kv_c, 16) || !aligned(k_pe, 4) || !aligned(cache, 16) || !aligned(slot_mapping, 8))
    return fail(DSA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  if (T == 0) return DSA_OK;
  dsa::launch_cache_insert(kv_c, kv_c_ld, k_pe, k_pe_ld, T, cache, kind, cache_scale,
                           slot_mapping, num_slots, stream);
  return launched(fn);
}

int dsa_launch_floor(int32_t workgroups, int32_t threads, hipStream_t stream) {
  const char* fn = "dsa_launch_floor";
  if (workgroups < 1) return fail(DSA_ERR_INVALID_ARG, "%s: workgroups=%d < 1", fn, workgroups);
  if (threads != 256 && threads != 512 && threads != 1024)
    return fail(DSA_ERR_INVALID_ARG, "%s: threads=%d not 256, 512 or 1024", fn, threads);
  dsa::launch_floor(workgroups, threads, stream);
  return launched(fn);
}

}  // extern "C"
