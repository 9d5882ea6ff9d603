// Sparse multi-query latent attention (MLA) decode over the selected latent
// rows of one shard, returning the partial output and a base-e LSE.
//
// What is computed (PR #52046 report, 关键源码片段: `forward_mqa(q, kv_cache,
// ...) -> (attn_out, lse)`, the cache entry being kv_c (512) followed by the
// roped k_pe (64); PR #46076 report, 实现拆解 item 5 / 评论区精华: the DCP
// reducer needs the LSE in base e):
//   s_j = sm_scale * q . K_j (576 wide), out = softmax(s) V, V_j = K_j[0:512],
//   lse = ln sum_j exp(s_j).
//
// How (gfx950):
//  - a workgroup = 4 waves = 64 heads of one (shard, row); each wave owns 16
//    heads, holds their q as MFMA B-operand fragments in VGPRs (72 regs) and
//    their output (512 x 16, fp32) in 32 MFMA accumulators;
//  - the selected latent rows are gathered 32 tokens at a time from the paged
//    pool into LDS (row-major for the score product, and the first 512 columns
//    also transposed, token-contiguous, for the value product), prefetched one
//    tile ahead in registers;
//  - scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_bf16: the accumulator layout then gives each lane 8
//    tokens of ONE head, exactly the B-operand fragment the value product
//    O^T += V^T P^T needs — no cross-lane shuffle of P;
//  - online softmax in base 2 (v_exp_f32 is 2^x): scores are pre-scaled by
//    log2(e); the final lse is (m + log2 l) * ln 2;
//  - fp8 e4m3 entries are widened to bf16 exactly (e4m3 is a subset of bf16)
//    and the per-tensor scale is folded into the score scale and the output.
#include "launchers.h"

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

constexpr int kAttnThreads = 256;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerBlock = 64;
constexpr int kTile = 32;                 // tokens per LDS tile
constexpr int kKStride = kLatent + 8;     // bf16 elements per key row in LDS
constexpr int kVtStride = kTile + 8;      // bf16 elements per transposed value row
constexpr int kQSteps = kLatent / 32;     // 18 MFMA k-steps over 576
constexpr int kOBlocks = kValue / 16;     // 32 accumulator blocks of 16 features
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// e4m3 code (low byte) -> bf16 bits, exact.
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t b) {
  const uint32_t s = (b & 0x80u) << 8;
  const uint32_t em = b & 0x7fu;
  if (em == 0x7fu) return s | 0x7fc0u;                      // NaN
  const uint32_t e = em >> 3, m = em & 7u;
  if (e) return s | ((e + 120u) << 7) | (m << 4);
  if (m == 0) return s;
  const float f = (float)m * 0.001953125f;                  // m * 2^-9, exact
  return s | (__float_as_uint(f) >> 16);
}

template <bool FP8>
__global__ __launch_bounds__(kAttnThreads, 1) void sparse_mla_decode_kernel(
    const uint16_t* __restrict__ q, int rows, int heads, const void* __restrict__ cache,
    const float* __restrict__ cache_scale, int64_t num_slots, const int* __restrict__ slots,
    const int* __restrict__ counts, int k, float sm_scale, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kTile * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[kValue * kVtStride];
  __shared__ int s_slot[2][kTile];

  // x = row, y = part, z = head group: the head groups of one (row, part)
  // read the same latent rows and sit rows*parts workgroup ids apart, which
  // keeps them on one XCD (and its L2) when rows*parts is a multiple of 8.
  const int row = blockIdx.x;
  const int part = blockIdx.y;
  const int hg = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int h0 = hg * kHeadsPerBlock + wave * kHeadsPerWave;
  const bool active = h0 < heads;

  const int* my_slots = slots + ((int64_t)part * rows + row) * k;
  int cnt = counts ? counts[(int64_t)part * rows + row] : k;
  cnt = cnt < 0 ? 0 : (cnt > k ? k : cnt);
  const float kv_scale = FP8 ? cache_scale[0] : 1.0f;
  const float qk_scale = sm_scale * kv_scale * kLog2e;

  // q fragments (B operand of S^T = K Q^T): head h0 + l16, features
  // 32*kk + 8*grp .. +8
  bf16x8_t qf[kQSteps];
  if (active) {
    const uint16_t* qp = q + ((int64_t)row * heads + h0 + l16) * kLatent + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < kQSteps; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * kk);
  }

  f32x4_t o[kOBlocks];
#pragma unroll
  for (int mb = 0; mb < kOBlocks; ++mb) o[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- gather plumbing ----------------------------------------------------
  // bf16: a tile is 32 rows x 72 16-byte chunks = 2304 chunks, 9 per thread.
  // fp8 : 32 rows x 36 16-byte chunks (16 codes each) = 1152, 4.5 per thread.
  constexpr int kChunksPerRow = FP8 ? kLatent / 16 : kLatent / 8;
  constexpr int kChunks = kTile * kChunksPerRow;
  constexpr int kPerThread = (kChunks + kAttnThreads - 1) / kAttnThreads;
  uint4 pre[kPerThread];
  const uint8_t* cache8 = reinterpret_cast<const uint8_t*>(cache);
  const uint16_t* cache16 = reinterpret_cast<const uint16_t*>(cache);

  auto load_slots = [&](int t0, int buf) {
    if (tid < kTile) {
      const int t = t0 + tid;
      int s = -1;
      if (t < cnt) {
        s = my_slots[t];
        if (s < 0 || (int64_t)s >= num_slots) s = -1;
      }
      s_slot[buf][tid] = s;
    }
  };
  auto fetch = [&](int buf) {
#pragma unroll
    for (int it = 0; it < kPerThread; ++it) {
      const int c = it * kAttnThreads + tid;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (c < kChunks) {
        const int tok = c / kChunksPerRow;
        const int piece = c % kChunksPerRow;
        const int s = s_slot[buf][tok];
        if (s >= 0) {
          if constexpr (FP8)
            v = *reinterpret_cast<const uint4*>(cache8 + (int64_t)s * kLatent + piece * 16);
          else
            v = *reinterpret_cast<const uint4*>(cache16 + (int64_t)s * kLatent + piece * 8);
        }
      }
      pre[it] = v;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < kPerThread; ++it) {
      const int c = it * kAttnThreads + tid;
      if (c >= kChunks) break;
      const int tok = c / kChunksPerRow;
      const int piece = c % kChunksPerRow;
      if constexpr (FP8) {
        const uint32_t w[4] = {pre[it].x, pre[it].y, pre[it].z, pre[it].w};
        uint32_t h[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) h[e] = e4m3_to_bf16_bits((w[e >> 2] >> (8 * (e & 3))) & 0xffu);
        uint4 lo4 = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                               h[6] | (h[7] << 16));
        uint4 hi4 = make_uint4(h[8] | (h[9] << 16), h[10] | (h[11] << 16),
                               h[12] | (h[13] << 16), h[14] | (h[15] << 16));
        uint16_t* dst = s_k + tok * kKStride + piece * 16;
        *reinterpret_cast<uint4*>(dst) = lo4;
        *reinterpret_cast<uint4*>(dst + 8) = hi4;
        if (piece * 16 < kValue) {
#pragma unroll
          for (int e = 0; e < 16; ++e) s_vt[(piece * 16 + e) * kVtStride + tok] = (uint16_t)h[e];
        }
      } else {
        *reinterpret_cast<uint4*>(s_k + tok * kKStride + piece * 8) = pre[it];
        if (piece * 8 < kValue) {
          const uint32_t w[4] = {pre[it].x, pre[it].y, pre[it].z, pre[it].w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            s_vt[(piece * 8 + e) * kVtStride + tok] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  };

  // ---- main loop over tiles of 32 selected tokens -------------------------
  if (cnt > 0) {
    load_slots(0, 0);
    __syncthreads();
    fetch(0);
  }
  for (int t0 = 0; t0 < cnt; t0 += kTile) {
    const int buf = (t0 / kTile) & 1;
    store_tile();
    __syncthreads();                       // tile in LDS; slot list of buf final
    const int t_next = t0 + kTile;
    if (t_next < cnt) load_slots(t_next, buf ^ 1);
    __syncthreads();
    if (t_next < cnt) fetch(buf ^ 1);      // overlaps with the math below

    if (active) {
      // S^T for two 16-token blocks; M-block b row rho <-> tile token
      // 8*(rho/4) + 4*b + rho%4, so lane (grp) ends up with tokens 8*grp..+8.
      f32x4_t sacc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        sacc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int tok = 8 * (l16 >> 2) + 4 * b + (l16 & 3);
        const uint16_t* kp = s_k + tok * kKStride + 8 * grp;
#pragma unroll
        for (int kk = 0; kk < kQSteps; ++kk) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kp + 32 * kk);
          sacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], sacc[b], 0, 0, 0);
        }
      }
      // lane holds head h0 + l16, tokens 8*grp + e (e = 4*b + i)
      float sv[8];
      float mt = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = 8 * grp + e;
        const bool ok = (t0 + tok < cnt) && (s_slot[buf][tok] >= 0);
        sv[e] = ok ? sacc[e >> 2][e & 3] * qk_scale : -INFINITY;
        mt = fmaxf(mt, sv[e]);
      }
      mt = max_over_groups(mt);
      const float m_new = fmaxf(m_run, mt);
      const float base = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
      u16x8_t pb;
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = exp2f(sv[e] - base);
        pb[e] = f32_to_bf16(p);
        ls += p;                           // the denominator keeps fp32 p
      }
      ls = sum_over_groups(ls);
      l_run = l_run * alpha + ls;
      m_run = m_new;
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pb);
#pragma unroll
      for (int mb = 0; mb < kOBlocks; ++mb) {
        o[mb] *= alpha;
        const uint16_t* vp = s_vt + (16 * mb + l16) * kVtStride + 8 * grp;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vp);
        o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, o[mb], 0, 0, 0);
      }
    }
    __syncthreads();                       // LDS tile free for the next store
  }

  // ---- epilogue -------------------------------------------------------------
  if (active) {
    const float inv = l_run > 0.f ? kv_scale / l_run : 0.f;
    uint16_t* op = out + (((int64_t)part * rows + row) * heads + h0 + l16) * kValue + 4 * grp;
#pragma unroll
    for (int mb = 0; mb < kOBlocks; ++mb) {
      const uint2 v = make_uint2(pack_bf16x2(o[mb][0] * inv, o[mb][1] * inv),
                                 pack_bf16x2(o[mb][2] * inv, o[mb][3] * inv));
      *reinterpret_cast<uint2*>(op + 16 * mb) = v;
    }
    if (grp == 0) {
      const float lv = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
      lse[((int64_t)part * rows + row) * heads + h0 + l16] = lv;
    }
  }
}

int launch_sparse_mla_decode(const void* q, int rows, int heads, const void* cache,
                             bool fp8, const float* cache_scale, int64_t num_slots,
                             const int* slots, const int* counts, int k, int n_parts,
                             float sm_scale, void* out, float* lse, hipStream_t stream) {
  dim3 grid(rows, n_parts, (heads + kHeadsPerBlock - 1) / kHeadsPerBlock);
  const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q);
  uint16_t* o16 = reinterpret_cast<uint16_t*>(out);
  if (fp8) {
    hipLaunchKernelGGL(sparse_mla_decode_kernel<true>, grid, dim3(kAttnThreads), 0, stream, q16,
                       rows, heads, cache, cache_scale, num_slots, slots, counts, k, sm_scale,
                       o16, lse);
  } else {
    hipLaunchKernelGGL(sparse_mla_decode_kernel<false>, grid, dim3(kAttnThreads), 0, stream,
                       q16, rows, heads, cache, cache_scale, num_slots, slots, counts, k,
                       sm_scale, o16, lse);
  }
  return 0;
}

}  // namespace dsa
