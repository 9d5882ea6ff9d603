// Fused RMSNorm (kv_c, 512) + interleaved-pair RoPE (k_pe, 64), materialised
// and/or inserted into the latent cache.
//
// What is computed (PR #52046 report, 实现拆解 item 1 and 关键源码片段,
// `_fused_norm_rope_kernel` branch pid == 1): y = RMSNorm(kv_c) * w; for pair
// i, (x1, x2) = (k_pe[2i], k_pe[2i+1]), r1 = x1 cos - x2 sin, r2 = x2 cos +
// x1 sin, stored interleaved; outputs are written when given (materialise),
// and the cache entry [y | r] at slot_mapping[t] when a mapping is given
// (fp8: value / scale -> e4m3).  The insert takes the materialised bf16
// values, so "materialise then insert" and the fused insert agree bit for bit.
//
// How: one wave per token; each lane owns 8 contiguous kv_c elements (16-byte
// load) and lanes 0..31 one rope pair; the sum of squares is a wave
// butterfly; math in fp32; stores are 16 bytes (bf16) / 8 bytes (fp8).
//
// The indexer-key branch (the same kernel's pid == 0 branch: PR #52046
// report, 实现拆解 item 1) runs in the same launch, one wave per token on the
// second grid row: RMSNorm over the 128-wide key with its own weight, RoPE
// over its last 64 dimensions in interleaved pairs (same table and position
// as the latent branch), materialised when index_k_out is given, and written
// into the fp8 indexer cache (e4m3(bf16 value / scale)) only when both that
// cache and the slot mapping are given.  Each lane holds 2 elements; lanes
// 32..63 hold the rotary pairs.
//
// cache_insert_kernel writes already materialised rows (the K rows that the
// sequence-sharded (PCP) path gathers from every rank before the update of
// its replicated cache: PR #52046 report, 关键源码片段, `do_kv_cache_update`
// after `maybe_gather_mla_latent_cache_inputs`) through the same insert
// code, so materialise + gather + insert equals the fused insert bit for bit.
#include "launchers.h"

namespace dsa {

constexpr int kNormThreads = 256;  // 4 tokens per block
constexpr int kIndexDim = 128;     // indexer key width

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Writes one cache entry [y | r] (8 kv_c values per lane; lanes 0..31 one
// rope pair): bf16 as is, fp8 as e4m3(value / scale).
template <int CACHE>
__device__ __forceinline__ void insert_row(int lane, const uint16_t (&y)[8], uint16_t r1b,
                                           uint16_t r2b, void* __restrict__ cache,
                                           const float* __restrict__ cache_scale, int64_t slot) {
  if constexpr (CACHE == 1) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(cache) + slot * kLatent;
    *reinterpret_cast<uint4*>(dst + 8 * lane) =
        make_uint4(y[0] | ((uint32_t)y[1] << 16), y[2] | ((uint32_t)y[3] << 16),
                   y[4] | ((uint32_t)y[5] << 16), y[6] | ((uint32_t)y[7] << 16));
    if (lane < kRope / 2)
      *reinterpret_cast<uint32_t*>(dst + kValue + 2 * lane) = (uint32_t)r1b | ((uint32_t)r2b << 16);
  } else {
    const float sc = cache_scale[0];
    uint8_t* dst = reinterpret_cast<uint8_t*>(cache) + slot * kLatent;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) lo |= f32_to_e4m3(bf16_to_f32(y[e]) / sc) << (8 * e);
#pragma unroll
    for (int e = 0; e < 4; ++e) hi |= f32_to_e4m3(bf16_to_f32(y[4 + e]) / sc) << (8 * e);
    *reinterpret_cast<uint2*>(dst + 8 * lane) = make_uint2(lo, hi);
    if (lane < kRope / 2) {
      const uint32_t c1 = f32_to_e4m3(bf16_to_f32(r1b) / sc);
      const uint32_t c2 = f32_to_e4m3(bf16_to_f32(r2b) / sc);
      *reinterpret_cast<uint16_t*>(dst + kValue + 2 * lane) = (uint16_t)(c1 | (c2 << 8));
    }
  }
}

// The indexer-key row of token t at position pos (see the header comment).
__device__ __forceinline__ void index_row(int t, int pos, int lane, const IndexerArgs& ix,
                                          const float* __restrict__ cos_sin,
                                          const int64_t* __restrict__ slot_mapping) {
  const uint32_t xv = *reinterpret_cast<const uint32_t*>(ix.k + (int64_t)t * ix.ld + 2 * lane);
  const uint32_t wv = *reinterpret_cast<const uint32_t*>(ix.w + 2 * lane);
  const float x0 = bf16_to_f32((uint16_t)(xv & 0xffffu));
  const float x1 = bf16_to_f32((uint16_t)(xv >> 16));
  const float ss = wave_sum(x0 * x0 + x1 * x1);
  const float inv_rms = 1.0f / sqrtf(ss / (float)kIndexDim + ix.eps);
  float y0 = x0 * inv_rms * bf16_to_f32((uint16_t)(wv & 0xffffu));
  float y1 = x1 * inv_rms * bf16_to_f32((uint16_t)(wv >> 16));
  if (lane >= (kIndexDim - kRope) / 2) {   // rotary pair i = lane - 32
    const int i = lane - (kIndexDim - kRope) / 2;
    const float c = cos_sin[(int64_t)pos * kRope + i];
    const float s = cos_sin[(int64_t)pos * kRope + kRope / 2 + i];
    const float r0 = y0 * c - y1 * s;
    const float r1 = y1 * c + y0 * s;
    y0 = r0;
    y1 = r1;
  }
  const uint16_t b0 = f32_to_bf16(y0), b1 = f32_to_bf16(y1);
  if (ix.out)
    *reinterpret_cast<uint32_t*>(ix.out + (int64_t)t * kIndexDim + 2 * lane) =
        (uint32_t)b0 | ((uint32_t)b1 << 16);
  if (ix.cache && slot_mapping) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= ix.num_slots) return;
    const float sc = ix.scale[0];
    const uint32_t c0 = f32_to_e4m3(bf16_to_f32(b0) / sc);
    const uint32_t c1 = f32_to_e4m3(bf16_to_f32(b1) / sc);
    *reinterpret_cast<uint16_t*>(ix.cache + slot * kIndexDim + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
  }
}

// CACHE: 0 = no insert, 1 = bf16 cache, 2 = fp8 e4m3 cache (latent branch).
// Grid row blockIdx.y + role0: 0 = latent branch, 1 = indexer-key branch.
template <int CACHE>
__global__ __launch_bounds__(kNormThreads) void fused_rmsnorm_rope_kernel(
    const uint16_t* __restrict__ kv_c, int64_t kv_ld, const uint16_t* __restrict__ k_pe,
    int64_t pe_ld, int T, const uint16_t* __restrict__ w, float eps,
    const float* __restrict__ cos_sin, int n_pos, const int* __restrict__ positions,
    uint16_t* __restrict__ kv_out, uint16_t* __restrict__ pe_out, void* __restrict__ cache,
    const float* __restrict__ cache_scale, const int64_t* __restrict__ slot_mapping,
    int64_t num_slots, IndexerArgs ix, int role0) {
  const int t = blockIdx.x * (kNormThreads / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // per-wave early out; no block barriers below
  const int lane = lane_id();
  const int pos = positions[t];
  if (pos < 0 || pos >= n_pos) return;
  if (role0 + (int)blockIdx.y == 1) {
    index_row(t, pos, lane, ix, cos_sin, slot_mapping);
    return;
  }

  // RMSNorm over 512
  const uint4 xv = *reinterpret_cast<const uint4*>(kv_c + (int64_t)t * kv_ld + 8 * lane);
  const uint4 wv = *reinterpret_cast<const uint4*>(w + 8 * lane);
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
  const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
  float x[8], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = bf16_to_f32((uint16_t)(xw[e >> 1] >> (16 * (e & 1))));
    ss += x[e] * x[e];
  }
  ss = wave_sum(ss);
  const float inv_rms = 1.0f / sqrtf(ss / (float)kValue + eps);
  uint16_t y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float we = bf16_to_f32((uint16_t)(ww[e >> 1] >> (16 * (e & 1))));
    y[e] = f32_to_bf16(x[e] * inv_rms * we);
  }

  // RoPE over 64 (lanes 0..31: pair i = lane)
  uint16_t r1b = 0, r2b = 0;
  if (lane < kRope / 2) {
    const uint32_t pr = *reinterpret_cast<const uint32_t*>(k_pe + (int64_t)t * pe_ld + 2 * lane);
    const float x1 = bf16_to_f32((uint16_t)(pr & 0xffffu));
    const float x2 = bf16_to_f32((uint16_t)(pr >> 16));
    const float c = cos_sin[(int64_t)pos * kRope + lane];
    const float s = cos_sin[(int64_t)pos * kRope + kRope / 2 + lane];
    r1b = f32_to_bf16(x1 * c - x2 * s);
    r2b = f32_to_bf16(x2 * c + x1 * s);
  }

  const uint4 yv = make_uint4(y[0] | ((uint32_t)y[1] << 16), y[2] | ((uint32_t)y[3] << 16),
                              y[4] | ((uint32_t)y[5] << 16), y[6] | ((uint32_t)y[7] << 16));
  const uint32_t rv = (uint32_t)r1b | ((uint32_t)r2b << 16);
  if (kv_out) *reinterpret_cast<uint4*>(kv_out + (int64_t)t * kValue + 8 * lane) = yv;
  if (pe_out && lane < kRope / 2)
    *reinterpret_cast<uint32_t*>(pe_out + (int64_t)t * kRope + 2 * lane) = rv;

  if constexpr (CACHE != 0) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;
    insert_row<CACHE>(lane, y, r1b, r2b, cache, cache_scale, slot);
  }
}

// CACHE: 1 = bf16 cache, 2 = fp8 e4m3 cache
template <int CACHE>
__global__ __launch_bounds__(kNormThreads) void cache_insert_kernel(
    const uint16_t* __restrict__ kv_c, int64_t kv_ld, const uint16_t* __restrict__ k_pe,
    int64_t pe_ld, int T, void* __restrict__ cache, const float* __restrict__ cache_scale,
    const int64_t* __restrict__ slot_mapping, int64_t num_slots) {
  const int t = blockIdx.x * (kNormThreads / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int lane = lane_id();
  const uint4 xv = *reinterpret_cast<const uint4*>(kv_c + (int64_t)t * kv_ld + 8 * lane);
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
  uint16_t y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (uint16_t)(xw[e >> 1] >> (16 * (e & 1)));
  uint16_t r1b = 0, r2b = 0;
  if (lane < kRope / 2) {
    const uint32_t pr = *reinterpret_cast<const uint32_t*>(k_pe + (int64_t)t * pe_ld + 2 * lane);
    r1b = (uint16_t)(pr & 0xffffu);
    r2b = (uint16_t)(pr >> 16);
  }
  insert_row<CACHE>(lane, y, r1b, r2b, cache, cache_scale, slot);
}

int launch_cache_insert(const void* kv_c, int64_t kv_ld, const void* k_pe, int64_t pe_ld, int T,
                        void* cache, int cache_kind, const float* cache_scale,
                        const int64_t* slot_mapping, int64_t num_slots, hipStream_t stream) {
  const int wpb = kNormThreads / kWave;
  dim3 grid((T + wpb - 1) / wpb);
  auto a0 = reinterpret_cast<const uint16_t*>(kv_c);
  auto a1 = reinterpret_cast<const uint16_t*>(k_pe);
  if (cache_kind == 1)
    hipLaunchKernelGGL(cache_insert_kernel<1>, grid, dim3(kNormThreads), 0, stream, a0, kv_ld, a1,
                       pe_ld, T, cache, cache_scale, slot_mapping, num_slots);
  else
    hipLaunchKernelGGL(cache_insert_kernel<2>, grid, dim3(kNormThreads), 0, stream, a0, kv_ld, a1,
                       pe_ld, T, cache, cache_scale, slot_mapping, num_slots);
  return 0;
}

int launch_fused_rmsnorm_rope(const void* kv_c, int64_t kv_ld, const void* k_pe, int64_t pe_ld,
                              int T, const void* w, float eps, const float* cos_sin, int n_pos,
                              const int* positions, void* kv_out, void* pe_out, void* cache,
                              int cache_kind, const float* cache_scale,
                              const int64_t* slot_mapping, int64_t num_slots, bool latent,
                              const IndexerArgs& ix, bool indexer, hipStream_t stream) {
  const int wpb = kNormThreads / kWave;
  // grid rows: the latent branch and/or the indexer-key branch
  const int role0 = latent ? 0 : 1;
  dim3 grid((T + wpb - 1) / wpb, (latent ? 1 : 0) + (indexer ? 1 : 0));
  auto a0 = reinterpret_cast<const uint16_t*>(kv_c);
  auto a1 = reinterpret_cast<const uint16_t*>(k_pe);
  auto a2 = reinterpret_cast<const uint16_t*>(w);
  auto o0 = reinterpret_cast<uint16_t*>(kv_out);
  auto o1 = reinterpret_cast<uint16_t*>(pe_out);
#define DSA_LAUNCH_NORM(C)                                                                   \
  hipLaunchKernelGGL(fused_rmsnorm_rope_kernel<C>, grid, dim3(kNormThreads), 0, stream, a0,  \
                     kv_ld, a1, pe_ld, T, a2, eps, cos_sin, n_pos, positions, o0, o1, cache, \
                     cache_scale, slot_mapping, num_slots, ix, role0)
  if (cache_kind == 0) DSA_LAUNCH_NORM(0);
  else if (cache_kind == 1) DSA_LAUNCH_NORM(1);
  else DSA_LAUNCH_NORM(2);
#undef DSA_LAUNCH_NORM
  return 0;
}

}  // namespace dsa
