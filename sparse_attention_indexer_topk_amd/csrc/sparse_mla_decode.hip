// Sparse multi-query latent attention (MLA) decode over the selected latent
// rows of one shard, returning the partial output and a base-e LSE.
//
// What is computed (PR #52046 report, 关键源码片段: `forward_mqa(q, kv_cache,
// ...) -> (attn_out, lse)`, a cache entry being kv_c (512) followed by the
// roped k_pe (64); PR #46076 report, 实现拆解 item 5 / 评论区精华: the DCP
// reducer needs the LSE in base e):
//   s_j = sm_scale * q . K_j (576 wide), out = softmax(s) V, V_j = K_j[0:512],
//   lse = ln sum_j exp(s_j).
//
// How (gfx950, one workgroup = 8 waves = 128 heads of one (row, part, split)):
//  - waves work in pairs; a pair owns 32 heads.  Member u of a pair computes
//    the partial scores over features [288u, 288u + 288) with q in VGPRs as
//    the B operand of v_mfma_f32_32x32x16_bf16 (18 k-steps, 72 VGPRs); the
//    pair swaps its fp32 partials through LDS so both hold the full scores,
//    then member u accumulates output features [256u, 256u + 256) (8 blocks
//    of 32 x 32 fp32 = 128 accumulators).  That keeps a wave under 256
//    registers (two waves per SIMD) while the key tile enters LDS once for
//    all 128 heads;
//  - the part's slot list is staged once in LDS; the selected latent rows are
//    gathered 32 tokens per tile straight from HBM into LDS with
//    global_load_lds_dwordx4 (no register staging; a uniform base plus a
//    32-bit offset per lane when the pool spans less than 4 GiB) through a
//    3-stage ring: tiles t+1 and t+2 are in flight while tile t is consumed,
//    and a stage is reused only after the barrier that follows its last
//    reader; two barriers per tile (tile arrival, score exchange);
//  - the value fragments of output block mb+1 are read while the MFMAs of
//    block mb run, and the score k-steps are left to the compiler's
//    scheduler, so that LDS latency overlaps MFMA work;
//  - the 16-byte chunks of a row are XOR-swizzled (swz_key) so that both the
//    score-operand reads and the value transpose reads are free of bank
//    conflicts;
//  - scores are computed transposed, S^T = K Q^T (rows = tokens), so the
//    accumulator gives each lane 16 tokens of ONE head — exactly the B
//    operand (P^T) of the value product O^T += V^T P^T;
//  - V^T fragments are read from the same row-major tile with
//    ds_read_b64_tr_b16 (LDS transpose read): no transposed copy of V;
//  - softmax in base 2 (v_exp_f32 computes 2^x) against a reference max
//    fixed by the first tile: probabilities may exceed 1 by up to 2^64, which
//    fp32 accumulators and bf16 operands hold exactly as well as values near
//    1, so the accumulators never need rescaling inside the loop.  A tile
//    whose max exceeds the reference by more than 2^64 (possible only for
//    extreme score ranges) restarts the workgroup's token list with the
//    raised reference — exact, and free of accumulator-wide VALU work in the
//    hot loop; the denominator sums fp32 probabilities; lse = (m + log2 l) ln 2;
//  - fp8 e4m3 caches are gathered raw (576 B/row) and widened to bf16 in LDS
//    with the hardware converter (exact: e4m3 is a subset of bf16); the
//    per-tensor scale is folded into the score scale and the output;
//  - split-K: `splits` workgroups share a part's token list, each emitting its
//    own partial; lse_combine merges them like shards;
//  - the epilogue stages each wave's normalised outputs in LDS and stores them
//    as 16-byte lanes covering whole 512-byte row halves.
#include "launchers.h"

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;

constexpr int kAttnThreads = 512;
constexpr int kAttnWaves = kAttnThreads / kWave;   // 8
constexpr int kHPW = 32;                       // heads per wave pair
constexpr int kHPB = kHPW * kAttnWaves / 2;    // heads per block (128)
constexpr int kTile = 32;                      // tokens per tile
constexpr int kStages = 3;                     // tiles in the LDS ring
constexpr int kRowB = kLatent * 2;             // bf16 row bytes (1152)
constexpr int kRowChunks = kRowB / 16;         // 72 16-byte chunks
constexpr int kTileB = kTile * kRowB;          // 36864 bytes
constexpr int kRowB8 = kLatent;                // fp8 row bytes (576)
constexpr int kTileB8 = kTile * kRowB8;        // 18432 bytes
constexpr int kQSteps = kLatent / 16 / 2;      // 18 per pair member
constexpr int kOBlocks = kValue / 32 / 2;      // 8 per pair member
constexpr int kMaxSel = 2048;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRestartSlack = 64.0f;         // log2 units
// epilogue staging: each wave's 32 heads x 256 bf16 outputs, rows padded by
// 8 bytes so that the row-strided 8-byte writes spread over the banks
constexpr int kEpiRow = kValue + 8;            // bytes per staged row (256 bf16 + pad)
constexpr int kEpiWaveB = kHPW * kEpiRow;
constexpr int kEpiB = kAttnWaves * kEpiWaveB;

// DMA instructions (64 lanes x 16 B) per tile, dealt round-robin to the waves
constexpr int kDmaBf16Total = kTileB / (16 * kWave);           // 36
constexpr int kDmaFp8Total = kTileB8 / (16 * kWave);           // 18

__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }
// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void lgkm_wait0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}
// byte offset of logical 16-byte chunk c of token row t inside a bf16 tile
__device__ __forceinline__ int swz_key(int t) {
  return ((t >> 1) & 1) | (((t ^ (t >> 2)) & 1) << 1) | (((t ^ (t >> 1) ^ (t >> 3)) & 1) << 2);
}
__device__ __forceinline__ int chunk_off(int t, int c) { return t * kRowB + ((c ^ swz_key(t)) << 4); }

template <bool FP8, bool OFF32>
__global__ __launch_bounds__(kAttnThreads) void sparse_mla_decode_kernel(
    const uint16_t* __restrict__ q, int rows, int heads, const uint8_t* __restrict__ cache,
    const float* __restrict__ cache_scale, int64_t num_slots, const int* __restrict__ slots,
    const int* __restrict__ counts, int k, int splits, float sm_scale,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int kRingB = FP8 ? kTileB8 : kTileB;
  constexpr int kDmaTotal = FP8 ? kDmaFp8Total : kDmaBf16Total;
  constexpr int kDmaMax = (kDmaTotal + kAttnWaves - 1) / kAttnWaves;
  constexpr int kConvB = FP8 ? kTileB : 0;
  constexpr int kXB = kAttnWaves * 4 * kWave * 16;
  constexpr int kMainB = kStages * kRingB + kConvB + kXB;
  constexpr int kSmemB = kMainB > kEpiB ? kMainB : kEpiB;
  __shared__ __attribute__((aligned(16))) uint8_t s_main[kSmemB];
  __shared__ int s_slot[kMaxSel];
  __shared__ int s_restart;
  uint8_t (*s_ring)[kRingB] = reinterpret_cast<uint8_t (*)[kRingB]>(s_main);
  uint8_t* s_conv = s_main + kStages * kRingB;
  float4 (*s_x)[4][kWave] =
      reinterpret_cast<float4 (*)[4][kWave]>(s_main + kStages * kRingB + kConvB);

  const int row = blockIdx.x;
  const int part = blockIdx.y / splits;
  const int split = blockIdx.y % splits;
  const int hg = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int pair = wave >> 1;
  const int u = wave & 1;         // pair member: feature half
  const int lane = lane_id();
  const int j32 = lane & 31;      // head column / token row of 32x32 operands
  const int g = lane >> 5;        // k-group of 32x32 operands
  const int h0 = hg * kHPB + pair * kHPW;
  const int head = h0 + j32;
  const bool pair_on = h0 < heads;
  const bool head_on = head < heads;
  const int out_part = blockIdx.y;

  // ---- this split's slice of the part's token list --------------------------
  int cnt = counts ? counts[(int64_t)part * rows + row] : k;
  cnt = cnt < 0 ? 0 : (cnt > k ? k : cnt);
  if (num_slots <= 0) cnt = 0;
  const int per = ((cnt + splits - 1) / splits + kTile - 1) / kTile * kTile;
  const int t_lo = split * per < cnt ? split * per : cnt;
  const int t_hi = t_lo + per < cnt ? t_lo + per : cnt;
  const int n_tok = t_hi - t_lo;
  const int ntiles = (n_tok + kTile - 1) / kTile;

  const int* my_slots = slots + ((int64_t)part * rows + row) * k;
  for (int i = tid; i < n_tok; i += kAttnThreads) {
    const int s = my_slots[t_lo + i];
    s_slot[i] = (s < 0 || (int64_t)s >= num_slots) ? -1 : s;
  }

  const float kv_scale = FP8 ? cache_scale[0] : 1.0f;
  const float qk_scale = sm_scale * kv_scale * kLog2e;

  // q fragments: head `head`, features 288*u + 16*kk + 8*g .. +8 (in flight
  // while the first tiles are requested)
  bf16x8_t qf[kQSteps];
  {
    const uint16_t* qp =
        q + ((int64_t)row * heads + (head_on ? head : 0)) * kLatent + 288 * u + 8 * g;
#pragma unroll
    for (int kk = 0; kk < kQSteps; ++kk) {
      u16x8_t v = *reinterpret_cast<const u16x8_t*>(qp + 16 * kk);
      if (!head_on) v = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      qf[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  f32x16_t o[kOBlocks];
#pragma unroll
  for (int mb = 0; mb < kOBlocks; ++mb)
#pragma unroll
    for (int a = 0; a < 16; ++a) o[mb][a] = 0.f;
  float m_ref = -INFINITY, l_part = 0.f;
  if (tid == 0) s_restart = 0;
  lgkm_wait0();
  bar();   // slot list and flag ready (q may still be in flight)

  // ---- lane-invariant LDS byte offsets inside a bf16 tile -------------------
  // scores: k-step kk of member u reads logical chunk 36u + g + 2kk of token
  // row j32 -> qk_off[kk % 4] + 128 * (kk / 4)
  int qk_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) qk_off[i] = chunk_off(j32, 36 * u + g + 2 * i);
  // values (transpose reads): 16-lane group G = lane/16 has k-group g = G/2
  // and feature half fs = G%2; inside it, source role sp = lane%16 reads
  // token row 16*ks + 8*h + 4*g + sp/4 at features 256u + 32mb + 16fs +
  // 4(sp%4) -> pv_off[mb % 2][h] + 16*ks*row + 128*(mb/2) (the swizzle key is
  // linear and ignores row bit 4, so only h changes the per-lane base)
  int pv_off[2][2];
  {
    const int sp = lane & 15, fs = (lane >> 4) & 1;
    const int trb = 4 * g + (sp >> 2);
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int feat = 256 * u + 32 * par + 16 * fs + 4 * (sp & 3);
        pv_off[par][h] = chunk_off(trb + 8 * h, feat >> 3) + (feat & 7) * 2;
      }
  }

  // ---- DMA issue of tile tt into its ring stage -------------------------------
  // instruction `ins` fills 64 consecutive 16-byte chunk slots of the stage;
  // instructions are dealt round-robin to the waves.  With OFF32 the source is
  // the uniform cache base plus a 32-bit byte offset (one VGPR per lane).
  auto issue = [&](int tt) {
    uint8_t* stage = s_ring[tt % kStages];
    const int tbase = tt * kTile;
#pragma unroll
    for (int jj = 0; jj < kDmaMax; ++jj) {
      const int ins = jj * kAttnWaves + wave;
      if (ins < kDmaTotal) {
        const int p = ins * kWave + lane;
        int t, off;
        if constexpr (FP8) {
          t = p / (kRowB8 / 16);
          off = (p % (kRowB8 / 16)) * 16;
        } else {
          t = p / kRowChunks;
          off = ((p % kRowChunks) ^ swz_key(t)) * 16;
        }
        const int ti = tbase + t < n_tok ? tbase + t : 0;
        const int s = max(s_slot[ti], 0);
        const uint8_t* src;
        if constexpr (OFF32)
          src = cache + (uint32_t)((uint32_t)s * (uint32_t)(FP8 ? kRowB8 : kRowB) + (uint32_t)off);
        else
          src = cache + (int64_t)s * (FP8 ? kRowB8 : kRowB) + off;
        __builtin_amdgcn_global_load_lds((const void*)src,
                                         (lds_void_ptr)(stage + ins * kWave * 16), 16, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // this wave's DMA instructions per tile
  const int my_dma = kDmaTotal / kAttnWaves + (wave < kDmaTotal % kAttnWaves ? 1 : 0);

  // Tiles 0 and 1 are requested before the loop; iteration tt waits for tile
  // tt, passes the barrier (after which every wave is done with tile tt-1),
  // requests tile tt+2 into tile tt-1's stage and computes tile tt.  A
  // restart request raised while computing tile tt is seen at the next
  // barrier: inside the loop at the next tile's arrival barrier, after the
  // last tile at the barrier below the loop.
  int tt = 0;
  int next_issue = 0;
  for (;;) {
  for (; tt < ntiles;) {
    // stages of tiles <= tt+1 are free before this barrier (only at the start
    // or after a restart is anything left to request here)
    while (next_issue < ntiles && next_issue <= tt + 1) issue(next_issue++);
    if (tt + 1 < ntiles) {
      if (my_dma == 5) vm_wait<5>();
      else if (my_dma == 4) vm_wait<4>();
      else if (my_dma == 3) vm_wait<3>();
      else vm_wait<2>();
    } else {
      vm_wait<0>();
    }
    lgkm_wait0();
    bar();   // tile tt visible; every wave is done with tile tt-1
    if (s_restart) {
      // a reference max moved by more than 2^64: drop the partial sums and
      // replay the token list (every wave, since the tile ring is shared)
      vm_wait<0>();
      bar();
      if (tid == 0) s_restart = 0;
#pragma unroll
      for (int mb = 0; mb < kOBlocks; ++mb)
#pragma unroll
        for (int a = 0; a < 16; ++a) o[mb][a] = 0.f;
      l_part = 0.f;
      __syncthreads();
      tt = 0;
      next_issue = 0;
      continue;
    }
    if (next_issue < ntiles) issue(next_issue++);   // tile tt+2, into tile tt-1's stage

    const uint8_t* tile = s_ring[tt % kStages];
    if constexpr (FP8) {
      // widen to the swizzled bf16 layout: 1152 chunks of 16 codes
      for (int c = tid; c < kTileB8 / 16; c += kAttnThreads) {
        const int t = c / (kRowB8 / 16);
        const int c8 = c % (kRowB8 / 16);            // features 16*c8 .. +16
        const uint4 raw = *reinterpret_cast<const uint4*>(tile + c * 16);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t h[8];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q4], 1.0f, false);
          const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q4], 1.0f, true);
          h[2 * q4] = __builtin_bit_cast(uint32_t, lo);
          h[2 * q4 + 1] = __builtin_bit_cast(uint32_t, hi);
        }
        *reinterpret_cast<uint4*>(s_conv + chunk_off(t, 2 * c8)) = make_uint4(h[0], h[1], h[2], h[3]);
        *reinterpret_cast<uint4*>(s_conv + chunk_off(t, 2 * c8 + 1)) =
            make_uint4(h[4], h[5], h[6], h[7]);
      }
      lgkm_wait0();
      bar();
      tile = s_conv;
    }

    // token validity of this tile as a wave-uniform bit mask
    const int tbase = tt * kTile;
    const uint64_t vmask =
        __ballot(lane < kTile && tbase + lane < n_tok && s_slot[tbase + (lane & 31)] >= 0);

    // ---- partial S^T = K Q^T over this member's 288 features -----------------
    f32x16_t sacc;
#pragma unroll
    for (int a = 0; a < 16; ++a) sacc[a] = 0.f;
    if (pair_on) {
      // k-step kk reads logical chunk c0 + 2*kk of token row j32; the swizzle
      // only permutes the low 3 chunk bits, so the address is one of 4
      // per-lane bases (kk % 4) plus 128 bytes per 4 k-steps
#pragma unroll
      for (int kk = 0; kk < kQSteps; ++kk) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(tile + qk_off[kk & 3] + 128 * (kk >> 2));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc, 0, 0, 0);
      }
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
        s_x[wave][a4][lane] = make_float4(sacc[4 * a4], sacc[4 * a4 + 1], sacc[4 * a4 + 2],
                                          sacc[4 * a4 + 3]);
    }
    lgkm_wait0();
    bar();                                           // partials visible
    if (pair_on) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 x = s_x[wave ^ 1][a4][lane];
        sacc[4 * a4] += x.x;
        sacc[4 * a4 + 1] += x.y;
        sacc[4 * a4 + 2] += x.z;
        sacc[4 * a4 + 3] += x.w;
      }
      // lane holds head `head`, tokens 8*(a/4) + 4*g + a%4 (same in both members)
      if (vmask != 0xffffffffull) {
        const uint32_t vm = (uint32_t)(vmask >> (4 * g));
#pragma unroll
        for (int a = 0; a < 16; ++a)
          if (!((vm >> (8 * (a >> 2) + (a & 3))) & 1u)) sacc[a] = -INFINITY;
      }
      float mt = sacc[0];
#pragma unroll
      for (int a = 1; a < 16; ++a) mt = fmaxf(mt, sacc[a]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, kWave)) * qk_scale;
      if (m_ref == -INFINITY) {
        m_ref = mt;
      } else if (__any(mt > m_ref + kRestartSlack)) {
        m_ref = fmaxf(m_ref, mt);
        if (lane == 0) s_restart = 1;
      }
      const float nm = (m_ref == -INFINITY) ? 0.f : -m_ref;
      bf16x8_t pf0, pf1;   // probabilities, rounded to nearest even by the hardware
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[a], qk_scale, nm));
        l_part += p;
        if (a < 8) pf0[a] = static_cast<__bf16>(p);
        else pf1[a - 8] = static_cast<__bf16>(p);
      }

      // ---- O^T += V^T P^T over this member's 256 output features --------------
      // V^T fragments come from the row-major tile through ds_read_b64_tr_b16:
      // 16-lane group G = lane/16 has k-group g = G/2 and feature half fs = G%2;
      // inside it, source role sp = lane%16 addresses token row
      // 8*(2*ks + h) + 4*g + sp/4 at features f + 16*fs + 4*(sp%4).
      auto vfrag = [&](int mb, int ks) {
        s16x4_t v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(
              tile + pv_off[mb & 1][h] + 16 * ks * kRowB + 128 * (mb >> 1)));
        return __builtin_bit_cast(bf16x8_t,
                                  __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8_t va0 = vfrag(0, 0), va1 = vfrag(0, 1);
#pragma unroll
      for (int mb = 0; mb < kOBlocks; ++mb) {
        bf16x8_t nb0 = va0, nb1 = va1;
        if (mb + 1 < kOBlocks) {   // next block's fragments in flight during these MFMAs
          nb0 = vfrag(mb + 1, 0);
          nb1 = vfrag(mb + 1, 1);
        }
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va0, pf0, o[mb], 0, 0, 0);
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va1, pf1, o[mb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        va0 = nb0;
        va1 = nb1;
      }
    }
    ++tt;
  }
  lgkm_wait0();
  bar();
  if (!s_restart) break;
  bar();
  if (tid == 0) s_restart = 0;
#pragma unroll
  for (int mb = 0; mb < kOBlocks; ++mb)
#pragma unroll
    for (int a = 0; a < 16; ++a) o[mb][a] = 0.f;
  l_part = 0.f;
  __syncthreads();
  tt = 0;
  next_issue = 0;
  }

  // ---- epilogue ---------------------------------------------------------------
  // Each wave stages its 32 heads x 256 normalised bf16 outputs row-major in
  // LDS (the tile ring is free: every wave passed the barrier after the last
  // tile), then stores them with 16-byte lanes, two 512-byte row halves per
  // instruction.
  const float l_tot = l_part + __shfl_xor(l_part, 32, kWave);
  const float inv = l_tot > 0.f ? kv_scale / l_tot : 0.f;
  uint8_t* stg = s_main + wave * kEpiWaveB;
  if (pair_on) {
#pragma unroll
    for (int mb = 0; mb < kOBlocks; ++mb)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint2 v = make_uint2(pack_bf16x2(o[mb][4 * b] * inv, o[mb][4 * b + 1] * inv),
                                   pack_bf16x2(o[mb][4 * b + 2] * inv, o[mb][4 * b + 3] * inv));
        *reinterpret_cast<uint2*>(stg + j32 * kEpiRow + (32 * mb + 8 * b + 4 * g) * 2) = v;
      }
  }
  lgkm_wait0();   // a wave reads back only what it wrote itself
  if (pair_on) {
    uint16_t* ob = out + (((int64_t)out_part * rows + row) * heads + h0) * kValue + 256 * u;
    const int half = lane >> 5, col = (lane & 31) * 16;
#pragma unroll
    for (int i = 0; i < kHPW / 2; ++i) {
      const int r = 2 * i + half;
      if (h0 + r < heads) {
        const uint4 v = *reinterpret_cast<const uint4*>(stg + r * kEpiRow + col);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(ob + (int64_t)r * kValue) + col) = v;
      }
    }
    if (head_on && g == 0 && u == 0) {
      const float lv = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
      lse[((int64_t)out_part * rows + row) * heads + head] = lv;
    }
  }
}

int launch_sparse_mla_decode(const void* q, int rows, int heads, const void* cache, bool fp8,
                             const float* cache_scale, int64_t num_slots, const int* slots,
                             const int* counts, int k, int n_parts, int splits, float sm_scale,
                             void* out, float* lse, hipStream_t stream) {
  dim3 grid(rows, n_parts * splits, (heads + kHPB - 1) / kHPB);
  const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q);
  const uint8_t* c8 = reinterpret_cast<const uint8_t*>(cache);
  uint16_t* o16 = reinterpret_cast<uint16_t*>(out);
  // 32-bit gather offsets when the whole pool lies within 4 GiB of its base
  const bool off32 = num_slots * (int64_t)(fp8 ? kRowB8 : kRowB) <= (int64_t)0xffffffffLL;
#define DSA_ATTN(F, O)                                                                       \
  hipLaunchKernelGGL((sparse_mla_decode_kernel<F, O>), grid, dim3(kAttnThreads), 0, stream,   \
                     q16, rows, heads, c8, cache_scale, num_slots, slots, counts, k, splits,  \
                     sm_scale, o16, lse)
  if (fp8) {
    if (off32) DSA_ATTN(true, true);
    else DSA_ATTN(true, false);
  } else {
    if (off32) DSA_ATTN(false, true);
    else DSA_ATTN(false, false);
  }
#undef DSA_ATTN
  return 0;
}

}  // namespace dsa
