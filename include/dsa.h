/*
 * dsa.h — C ABI of the MI355X (gfx950) DSA sparse-attention library.
 *
 * DeepSeek-V3.2-style sparse attention ("DSA") over a context-sharded KV
 * cache, as described by three vLLM pull-request reports:
 *   [A] "PR #46076 [Attention][DSA] support dcp for FLASHINFER_MLA_SPARSE"
 *   [B] "PR #40996 DCP supports hybrid attention"
 *   [C] "PR #52046" (DSV3.2 prefill context parallel, fused norm + RoPE)
 *
 * The decode-context-parallel (DCP) path runs, per step:
 *   dsa_fused_rmsnorm_rope (fp8 workload) -> dsa_topk_select (all shards)
 *   -> dsa_merge_candidates -> dsa_convert_index -> dsa_sparse_mla_decode
 *   -> dsa_lse_combine.
 * dsa_merge_convert runs the merge and the conversion as one launch.
 * All shards of one job live on one GPU as slices of one buffer.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All array pointers are DEVICE pointers (HIP global memory) unless noted.
 *   The caller owns every buffer; the library allocates nothing and keeps no
 *   state besides its code object and a thread-local error message.
 * - Every call only validates its host arguments and enqueues kernels on
 *   `stream` (0 = the null stream); nothing is synchronised.
 * - The return value is a dsa_status.  Validation happens before any HIP
 *   call, so an invalid call has no side effect.  dsa_last_error() returns a
 *   message for the last non-OK status of the calling thread.
 * - rows == 0 (or T == 0) is a successful no-op (as the attention layer
 *   returns early when there are no tokens, [C] 关键源码片段).
 * - Inputs and outputs must not alias.
 * - Device-resident values are clamped or skipped, never trusted for
 *   addressing: row bounds are clamped to [0, ctx], ids outside
 *   [0, id_bound), slots outside the pool and requests outside the table are
 *   ignored as described per call.  No call reads or writes outside the
 *   buffers its size arguments describe.
 *
 * Shard notation: S = num_shards, I = interleave.  Global token t lives on
 * shard owner(t) = (t / I) % S at local position local(t) = (t / (I*S))*I
 * + t % I ([A] 关键源码片段, `_dcp_localize_decode_seq_lens`: a rank owns the
 * positions whose (pos // interleave) % world equals its rank).  A call runs
 * the shards [shard_first, shard_first + shard_count); slice j of a
 * shard-sliced buffer belongs to shard shard_first + j.
 */
#ifndef DSA_H
#define DSA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1,       /* null pointer, bad size, bad shard range */
  DSA_ERR_UNSUPPORTED_K = -2,     /* k not in {512, 1024, 2048} */
  DSA_ERR_UNSUPPORTED_DTYPE = -3, /* dtype code not accepted by this call */
  DSA_ERR_HIP = -4                /* a HIP launch failed */
} dsa_status;

typedef enum { DSA_BF16 = 1, DSA_FP32 = 2, DSA_FP8_E4M3 = 3 } dsa_dtype;

#define DSA_LATENT_DIM 576  /* 512 kv_c + 64 rope */
#define DSA_VALUE_DIM 512
#define DSA_ROPE_DIM 64
#define DSA_INDEX_DIM 128   /* indexer key: 64 unrotated + 64 rotary dimensions */
#define DSA_MAX_SHARDS 16
#define DSA_MAX_ID (1 << 24) /* global ids travel as exact fp32 values */

/*
 * dsa_topk_select — per-shard stable top-K over fp32 indexer logits, with the
 * (score, global_id) candidate packing fused in.
 *
 * Source: [A] 关键源码片段 `_merge_dcp_topk_global` and 实现拆解 item 1: every
 * rank holds "the top-K positions in this rank's local KV shard", packs them
 * as (score, global_id) into a float32 [batch, topk, 2] buffer and
 * all-gathers along dim 1; `_assert_cutedsl_dcp_merge_supported` requires
 * fp32 logits, int32 indices and k in {512, 1024, 2048}.
 *
 * logits      [shard_count][rows][ld] fp32; slice j starts at
 *             logits + j*shard_stride.  Column l of shard r's slice is the
 *             logit of local position l (global token global(r, l)).
 *             Columns < local_count(ctx, r) must be readable: ld >= that.
 * row_starts  [rows] int32 global start of each row's valid range (NULL: 0)
 * row_ends    [rows] int32 global end, exclusive (NULL: ctx).  Both are
 *             clamped to [0, ctx]; shard r's valid local range is
 *             [local_count(start, r), local_count(end, r)).
 * local_idx   [shard_count][rows][k] int32 output (NULL: not written):
 *             the selected local positions, ascending, then -1.
 * cand        [rows][S*k][2] fp32 output (NULL: not written): shard r writes
 *             columns [r*k, (r+1)*k) — the all-gather, done in place — with
 *             (logit, global id) per selection in ascending order, then
 *             (-inf, -1.0).  Columns of shards outside the run are untouched.
 * Selection order: larger logit first; equal logits (-0.0 == +0.0) by
 * smaller position.  NaN ranks below every number.
 * Errors: INVALID_ARG (null logits, both outputs NULL, rows < 0, ctx outside
 * [0, 2^24], shard range, ld too small, negative strides), UNSUPPORTED_K.
 */
int dsa_topk_select(const float* logits, int64_t ld, int64_t shard_stride,
                    int32_t rows, int32_t ctx, const int32_t* row_starts,
                    const int32_t* row_ends, int32_t k, int32_t num_shards,
                    int32_t interleave, int32_t shard_first,
                    int32_t shard_count, int32_t* local_idx, float* cand,
                    hipStream_t stream);

/*
 * dsa_merge_candidates — stable global top-K over gathered candidates.
 *
 * Source: [A] 实现拆解 item 1 and 关键源码片段 (`stable_topk_from_gathered_
 * candidates(gathered, topk_tokens, out=topk_indices)`): select the global
 * top-K token ids from every rank's (score, global_id) pairs; -1 = padding.
 *
 * cand   [rows][n_cand][2] fp32 (score, id); an entry is valid when its id is
 *        an integer value in [0, id_bound).  Valid ids must be distinct
 *        within a row (true of dsa_topk_select output).
 * ids    [rows][k] int32 output: the min(k, #valid) best valid candidates'
 *        ids in ascending order, then -1.
 * Order: larger score first, equal scores by smaller id.
 * Errors: INVALID_ARG (null pointers, rows < 0, n_cand < 1 or > 16*k,
 * id_bound outside [1, 2^24]), UNSUPPORTED_K.
 */
int dsa_merge_candidates(const float* cand, int32_t rows, int32_t n_cand,
                         int32_t k, int32_t id_bound, int32_t* ids,
                         hipStream_t stream);

/*
 * dsa_convert_index — global token ids -> per-shard physical cache slots,
 * valid slots compacted to the front.
 *
 * Source: [A] 实现拆解 item 4 (`_convert_req_index_to_global_index_kernel`
 * with DCP_SIZE / DCP_RANK / DCP_INTERLEAVE and COMPACT_TO_FRONT): a rank
 * keeps the ids it owns, de-interleaves each to its local position, maps it
 * through its block table and packs the valid slots at the front.
 *
 * ids          [rows][k] int32 global ids (any order; < 0 = padding).
 * row_req      [rows] int32 request of each row (NULL: row i -> request i).
 *              Rows whose request is outside [0, num_reqs) get no slots.
 * block_table  [shard_count][num_reqs][bt_ld] int32 physical block ids;
 *              slice j at block_table + j*bt_shard_stride.
 * slots        [shard_count][rows][k] int32 output: for shard r, the ids it
 *              owns, in input order, as block_table[req][l / block_size] *
 *              block_size + l % block_size (l = local position), then -1.
 *              Ids whose block column is >= bt_ld are skipped.
 * counts       [shard_count][rows] int32 output (NULL: not written).
 * Errors: INVALID_ARG (null ids/block_table/slots, sizes, shard range,
 * block_size < 1), UNSUPPORTED_K.
 */
int dsa_convert_index(const int32_t* ids, int32_t rows, int32_t k,
                      const int32_t* row_req, int32_t num_reqs,
                      const int32_t* block_table, int64_t bt_ld,
                      int64_t bt_shard_stride, int32_t block_size,
                      int32_t num_shards, int32_t interleave,
                      int32_t shard_first, int32_t shard_count, int32_t* slots,
                      int32_t* counts, hipStream_t stream);

/*
 * dsa_merge_convert — dsa_merge_candidates followed by dsa_convert_index of
 * the merged ids, in one launch.
 *
 * Source: [A] 实现拆解 items 1 and 4 (the global merge of the gathered
 * candidates, then each rank's conversion of the merged ids to its compacted
 * local cache slots).  Every output equals what the two calls produce in
 * sequence with the same arguments; the merged ids stay on chip in between.
 *
 * cand, n_cand, k, id_bound  as for dsa_merge_candidates.
 * ids          [rows][k] int32 output as for dsa_merge_candidates (NULL: not
 *              written).
 * row_req, num_reqs, block_table, bt_ld, bt_shard_stride, block_size,
 * num_shards, interleave, shard_first, shard_count, slots, counts  as for
 *              dsa_convert_index.
 * Errors: the union of both calls' checks.
 */
int dsa_merge_convert(const float* cand, int32_t rows, int32_t n_cand, int32_t k,
                      int32_t id_bound, int32_t* ids, const int32_t* row_req,
                      int32_t num_reqs, const int32_t* block_table, int64_t bt_ld,
                      int64_t bt_shard_stride, int32_t block_size,
                      int32_t num_shards, int32_t interleave,
                      int32_t shard_first, int32_t shard_count, int32_t* slots,
                      int32_t* counts, hipStream_t stream);

/*
 * dsa_sparse_mla_decode — per-shard sparse multi-query latent attention.
 *
 * Source: [C] 关键源码片段 (`forward_mqa(q, kv_cache, ...) -> (attn_out,
 * lse)`; the cache entry is kv_c (512) followed by the roped k_pe (64));
 * [A] 实现拆解 item 5 and 评论区精华 "LSE 基数归一化": the returned LSE must be
 * base e for the DCP reducer (the NVIDIA backend returns base 2 and is
 * rescaled by ln 2).
 *
 * For part p, row i, head h over the first counts[p][i] slots J:
 *   s_j  = sm_scale * dot(q[i][h][0:576], K_j[0:576])
 *   lse  = ln sum_j exp(s_j)            (base e)
 *   out  = sum_j exp(s_j - lse) * K_j[0:512]
 * K_j is the latent entry at slot j: bf16, or e4m3 code * (*cache_scale).
 * A part with no (valid) slots writes out = 0 and lse = -inf.
 *
 * q            [rows][heads][576] bf16.
 * cache        [num_slots][576] latent pool (slot = block*block_size + off),
 *              bf16 or fp8 e4m3 per cache_dtype.
 * cache_scale  device fp32 scalar (fp8 only; may be NULL for bf16).
 * slots        [n_parts][rows][k] int32; counts [n_parts][rows] int32 (NULL:
 *              every entry up to k is examined).  Slots outside
 *              [0, num_slots) are skipped.
 * splits       split-K factor >= 1: each part's slot list is cut into
 *              `splits` consecutive pieces (multiples of 32 slots), each
 *              producing its own partial; partial p*splits + s belongs to
 *              part p.  All partials merge with dsa_lse_combine.
 * out          [n_parts*splits][rows][heads][512] output of out_dtype:
 *              DSA_BF16 (the path's format, round to nearest even) or
 *              DSA_FP32 (a checking mode: the same normalised values without
 *              the bf16 rounding).
 * lse          [n_parts*splits][rows][heads] fp32 output.
 * Errors: INVALID_ARG (null pointers, heads not a positive multiple of 16,
 * splits outside [1, 64], rows*n_parts*splits*ceil(heads/128) above
 * 2^31 - 1, sizes), UNSUPPORTED_K, UNSUPPORTED_DTYPE (cache not bf16/fp8,
 * out_dtype not bf16/fp32).
 */
int dsa_sparse_mla_decode(const void* q, int32_t rows, int32_t heads,
                          const void* cache, int32_t cache_dtype,
                          const float* cache_scale, int64_t num_slots,
                          const int32_t* slots, const int32_t* counts,
                          int32_t k, int32_t n_parts, int32_t splits,
                          float sm_scale, void* out, int32_t out_dtype,
                          float* lse, hipStream_t stream);

/*
 * dsa_lse_combine — LSE-weighted merge of per-shard partial attention.
 *
 * Source: [C] 关键源码片段 (`dcp_manager.combine(attn_out, lse, ...)` after
 * forward_mqa); [A] 评论区精华: the reducer expects base-e LSE.
 *   lse = ln sum_p exp(lse_p) over finite lse_p (-inf if none)
 *   out = sum_p exp(lse_p - lse) * out_p       (0 if none)
 *
 * part_out  [n_parts][rows][heads][dim] of part_dtype (DSA_BF16, or DSA_FP32
 *           for the attention's fp32 checking mode); part_lse
 *           [n_parts][rows][heads] fp32.
 * out       [rows][heads][dim] bf16 output; lse_out [rows][heads] fp32
 *           output (NULL: not written).
 * Errors: INVALID_ARG (null pointers, n_parts outside [1, 64], dim not a
 *         positive multiple of 8, sizes), UNSUPPORTED_DTYPE (part_dtype not
 *         bf16/fp32).
 */
int dsa_lse_combine(const void* part_out, int32_t part_dtype,
                    const float* part_lse, int32_t n_parts, int32_t rows,
                    int32_t heads, int32_t dim, void* out, float* lse_out,
                    hipStream_t stream);

/*
 * dsa_fused_rmsnorm_rope — RMSNorm over kv_c + interleaved-pair RoPE over
 * k_pe (the latent branch), and the same for the indexer key (the indexer
 * branch); each branch materialises and/or inserts into its cache.
 *
 * Source: [C] 实现拆解 item 1 and 关键源码片段 (`_fused_norm_rope_kernel`).
 * Latent branch (pid == 1): y = RMSNorm(kv_c) with weight w and epsilon; for
 * pair i, (x1, x2) = (k_pe[2i], k_pe[2i+1]), r1 = x1*cos - x2*sin, r2 = x2*cos
 * + x1*sin, stored back interleaved; the outputs are materialised when their
 * pointers are given, and the cache entry [y | r] is written at the slot when
 * a slot mapping and a cache are given (fp8: value / scale cast to e4m3).
 * Indexer branch (pid == 0): the indexer key is materialised into
 * index_k_out when given, and quantised to fp8 and written into the indexer
 * cache only when both index_cache and slot_mapping are given.  The call
 * returns at once, with nothing written, only when all three outputs
 * (kv_c_out, k_pe_out, index_k_out) and the slot mapping are NULL.
 *
 * The pages do not print the indexer branch's arithmetic; this library takes
 * the plainest reading of the latent branch: the key is 128 wide (64
 * unrotated dimensions, then a 64-dimension rotary part), RMSNorm over all
 * 128 with weight index_w and index_eps, then the same interleaved-pair RoPE
 * over the last 64 (same table and position), rounded once to bf16; the
 * indexer cache holds e4m3(bf16 value / *index_cache_scale) (nearest-even,
 * saturating at 448), 128 bytes per slot, at the latent branch's slots.
 *
 * kv_c [T][kv_c_ld] bf16 (first 512 used); k_pe [T][k_pe_ld] bf16 (first 64);
 * rms_w [512] bf16; cos_sin [n_pos][64] fp32 = cos(32) | sin(32) of each
 * position; positions [T] int32 (rows with a position outside [0, n_pos)
 * are left unwritten by both branches).
 * kv_c_out [T][512], k_pe_out [T][64] bf16 outputs (each NULL: not written).
 * cache [num_slots][576] bf16 or fp8 e4m3; cache_scale device fp32 scalar
 * (fp8); slot_mapping [T] int64 (NULL: no insert; entries < 0 or >=
 * num_slots are skipped).  Inserted values are the materialised bf16
 * values (fp8: e4m3(bf16 value / scale), nearest-even, saturating at 448).
 * index_k [T][index_k_ld] bf16 (first 128 used); index_w [128] bf16;
 * index_k_out [T][128] bf16 output (NULL: not written); index_cache
 * [index_num_slots][128] e4m3 (NULL: no indexer insert); index_cache_scale
 * device fp32 scalar.  The inputs of a branch are read only when it writes
 * something (the latent branch: kv_c_out, k_pe_out or a cache insert; the
 * indexer branch: index_k_out or an indexer-cache insert); both run in one
 * launch.
 * Errors: INVALID_ARG (a branch's null inputs, a slot mapping without any
 * cache, T < 0, lds < widths, misaligned pointers, missing scales),
 * UNSUPPORTED_DTYPE (latent cache not bf16/fp8 when inserting).
 */
int dsa_fused_rmsnorm_rope(const void* kv_c, int64_t kv_c_ld, const void* k_pe,
                           int64_t k_pe_ld, int32_t T, const void* rms_w,
                           float eps, const float* cos_sin, int32_t n_pos,
                           const int32_t* positions, void* kv_c_out,
                           void* k_pe_out, void* cache, int32_t cache_dtype,
                           const float* cache_scale,
                           const int64_t* slot_mapping, int64_t num_slots,
                           const void* index_k, int64_t index_k_ld,
                           const void* index_w, float index_eps,
                           void* index_k_out, void* index_cache,
                           const float* index_cache_scale,
                           int64_t index_num_slots, hipStream_t stream);

/*
 * dsa_cache_insert — write already materialised K rows into the latent cache.
 *
 * Source: [C] 关键源码片段 (the PCP branch of `_sparse_indexer_and_attn`):
 * with queries sharded by sequence the MLA cache is replicated, so the new K
 * rows every rank materialised are gathered (`maybe_gather_mla_latent_cache_
 * inputs`) and then written into each replica (`do_kv_cache_update` with the
 * cache dtype and k scale).  The values are written exactly as the insert of
 * dsa_fused_rmsnorm_rope writes its materialised rows, so materialise +
 * gather + insert equals the fused insert bit for bit.
 *
 * kv_c [T][kv_c_ld] bf16 (first 512), k_pe [T][k_pe_ld] bf16 (first 64):
 *              the materialised rows.
 * cache [num_slots][576] bf16 or fp8 e4m3 per cache_dtype; cache_scale device
 *              fp32 scalar (fp8): entries are e4m3(value / scale),
 *              nearest-even, saturating at 448.
 * slot_mapping [T] int64 (entries < 0 or >= num_slots are skipped).
 * Errors: INVALID_ARG (null pointers, T < 0, lds < widths, misaligned),
 * UNSUPPORTED_DTYPE.
 */
int dsa_cache_insert(const void* kv_c, int64_t kv_c_ld, const void* k_pe,
                     int64_t k_pe_ld, int32_t T, void* cache, int32_t cache_dtype,
                     const float* cache_scale, const int64_t* slot_mapping,
                     int64_t num_slots, hipStream_t stream);

/*
 * dsa_launch_floor — measurement helper, not a step of the path: launches a
 * kernel that returns at once with `workgroups` workgroups of `threads`
 * threads (256, 512 or 1024) on `stream`.  Its duration in a kernel trace is
 * the floor a path kernel of the same grid shape pays before doing any work.
 * Errors: INVALID_ARG (workgroups < 1, other thread counts).
 */
int dsa_launch_floor(int32_t workgroups, int32_t threads, hipStream_t stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* dsa_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
