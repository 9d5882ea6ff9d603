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
//  - score phase: each wave owns 16 heads over all 576 features; q (the B
//    operand of v_mfma_f32_16x16x32_bf16, 18 k-steps) stays in 72 VGPRs and
//    the key tile enters LDS once for all 128 heads;
//  - value phase, split by output features instead: wave w owns features
//    64w .. 64w+63 for all 128 heads (32 blocks of 16 x 16 fp32 in 128
//    VGPRs), so it reads 4 value fragments per tile and takes the P^T
//    operands of the 8 head blocks (1 KB each) that the score waves wrote to
//    LDS; per tile every wave reads the whole key tile once, but only an
//    eighth of the value tile;
//  - the selected latent rows are gathered 32 tokens per tile straight from
//    HBM into LDS with global_load_lds_dwordx4 (no register staging; a
//    uniform base plus a 32-bit offset per lane when the pool spans less
//    than 4 GiB); one barrier per tile;
//  - the gather lays a tile out in LDS as blocks of 16 tokens x 4 16-byte
//    chunks (1 KB), one gather instruction per block: each token's 64
//    contiguous bytes go to 4 consecutive lanes, which the memory path takes
//    as one request (a token per lane, the same bytes gathered 10 % slower),
//    and the 4 chunks of a token are permuted by its position so that the
//    score reads (16 tokens, one chunk) and the value transpose reads meet
//    no LDS bank conflict;
//  - scores are computed transposed, S^T = K Q^T (rows = tokens), so each
//    lane ends with 8 tokens of ONE head — with the token order inside the
//    k dimension permuted the same way on both operands, exactly the B
//    operand (P^T) of the value product O^T += V^T P^T, which the score wave
//    stores as is; V^T fragments come from the row-major tile through the
//    LDS transpose reads;
//  - softmax in base 2 (v_exp_f32 computes 2^x) against a reference max
//    fixed by the first tile: probabilities may exceed 1 by up to 2^64, which
//    fp32 accumulators and bf16 operands hold exactly as well as values near
//    1, so the accumulators never need rescaling inside the loop.  A tile
//    whose max exceeds the reference by more than 2^64 (possible only for
//    extreme score ranges) restarts the workgroup's token list with the
//    raised reference — exact, and free of accumulator-wide VALU work in the
//    hot loop; the denominator sums fp32 probabilities; lse = (m + log2 l) ln 2;
//  - fp8 e4m3 caches are gathered raw (576 B/row) into LDS; each wave reads
//    its operand codes straight from the raw tile (8 bytes per lane, the
//    value operand by an 8-bit transpose read) and widens them to bf16 in
//    registers with the hardware converter (exact: e4m3 is a subset of
//    bf16); the per-tensor scale is folded into the score scale and the
//    output;
//  - split-K: `splits` workgroups share a part's token list, each emitting its
//    own partial; lse_combine merges them like shards;
//  - the epilogue stages the normalised outputs in LDS and stores one whole
//    1 KB head row per instruction.
#include "launchers.h"

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef int i32x2_t __attribute__((ext_vector_type(2)));

constexpr int kAttnThreads = 512;
constexpr int kAttnWaves = kAttnThreads / kWave;   // 8
constexpr int kHPW = 16;                       // heads per wave
constexpr int kHPB = kHPW * kAttnWaves;        // heads per block (128)
constexpr int kTile = 32;                      // tokens per tile
constexpr int kRowB = kLatent * 2;             // bf16 row bytes (1152)
constexpr int kRowB8 = kLatent;                // fp8 row bytes (576)
constexpr int kQSteps = kLatent / 32;          // 18 k-steps of 32 features
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRestartSlack = 64.0f;         // log2 units
// epilogue staging: each wave's 16 heads x 512 bf16 outputs, rows padded by
// 16 bytes so that the row-strided 8-byte writes spread over the banks
constexpr int kEpiRow = kValue * 2 + 16;


__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }
// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void vm_wait_n(int n) {
  switch (n) {
    case 0: vm_wait<0>(); break;
    case 1: vm_wait<1>(); break;
    case 2: vm_wait<2>(); break;
    case 3: vm_wait<3>(); break;
    case 4: vm_wait<4>(); break;
    case 5: vm_wait<5>(); break;
    case 6: vm_wait<6>(); break;
    case 7: vm_wait<7>(); break;
    case 8: vm_wait<8>(); break;
    default: vm_wait<0>(); break;   // any other count: wait for everything
  }
}
__device__ __forceinline__ void lgkm_wait0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}
// compile-time loop: f(IntC<0>{}) .. f(IntC<N-1>{})
template <int I> struct IntC { static constexpr int value = I; };
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    static_for<N, I + 1>(f);
  }
}

// LDS reads of the tile operands, written as asm: issued as builtins right
// after the tile gathers (HBM -> LDS copies counted by vmcnt), the compiler
// guards them with a full vmcnt wait, because it cannot tell them from the
// copies still in flight, and the ring would drain every tile.  Each read is
// at LDS byte address addr + OFF; the caller waits for it with one of the
// lgkm_wait_* helpers below, which pass the destination registers through
// the wait so that no use can move above it.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <int OFF>
__device__ __forceinline__ u32x4_t lds_read_b128(uint32_t addr) {
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ i32x2_t lds_read_b64(uint32_t addr) {
  i32x2_t r;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ i32x2_t lds_read_tr16(uint32_t addr) {
  i32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ i32x2_t lds_read_tr8(uint32_t addr) {
  i32x2_t r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
// wait until at most N LDS operations of this wave are in flight
template <int N>
__device__ __forceinline__ void lgkm_wait_1(u32x4_t& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait_2(u32x4_t& a, u32x4_t& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait_2v(i32x2_t& a, i32x2_t& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait_4v(i32x2_t& a, i32x2_t& b, i32x2_t& c, i32x2_t& d) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "n"(N));
}

// 8 e4m3 codes -> 8 bf16 (exact: every e4m3 value is a bf16 value)
__device__ __forceinline__ bf16x8_t widen8(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const bf16x4_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4_t cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---- pipelining and LDS layout ----------------------------------------------
//  - iteration t: wait for tile t, barrier, request tile t + kAhead, values of
//    tile t-1 (its P^T written in iteration t-1, double-buffered by tile
//    parity), scores and softmax of tile t, P^T of tile t to LDS;
//  - the ring keeps features 0..511 of kAhead + 2 tiles (t-1 for values, t for
//    scores, kAhead in flight) and the rope features 512..575 of kAhead + 1;
//    bf16 tiles (36 KB) allow 2 tiles in flight in the 160 KB of LDS, raw fp8
//    tiles (18 KB) 3;
//  - the slot list is not staged whole: a ring of 8 tiles' entries is refilled
//    by an HBM->LDS copy of tile u + kAhead + 1's entries riding with the
//    gathers of tile u, so the wait for tile u covers it and its barrier
//    publishes it before tile u + kAhead + 1's gathers are issued;
//  - the output scale 1/l of each head is handed from its score wave to the
//    value waves through LDS after the last tile.
template <bool FP8>
struct AttnLayout {
  static constexpr int kRowBytes = FP8 ? kRowB8 : kRowB;    // 576 or 1152
  static constexpr int kBlocks = kRowBytes * kTile / 1024;  // 18 or 36 blocks of 1 KB
  static constexpr int kMainBlocks = kBlocks * 8 / 9;       // features 0..511: 16 or 32
  static constexpr int kMainB = kMainBlocks * 1024;
  static constexpr int kRopeB = (kBlocks - kMainBlocks) * 1024;
  static constexpr int kAhead = FP8 ? 3 : 2;                 // tiles in flight
  static constexpr int kMainStages = kAhead + 2;
  static constexpr int kRopeStages = kAhead + 1;
  static constexpr int kRingB = kMainStages * kMainB + kRopeStages * kRopeB;
  static constexpr int kStageB = kHPB * kEpiRow;             // epilogue staging
  static constexpr int kTilesB = kRingB > kStageB ? kRingB : kStageB;
  static constexpr int kDmaMax = (kBlocks + kAttnWaves - 1) / kAttnWaves;
  static constexpr int kRefill = kAhead + 1;                 // slot refill distance in tiles
  static constexpr int kKAhead = FP8 ? 3 : 2;                // key k-steps read ahead
};
constexpr int kPB = kTile * kHPB * 2;           // P^T of one tile, 128 heads (8 KB)
constexpr int kSlotRing = 8;                    // tiles of slot entries held in LDS
constexpr int kSlotInit = 4;                    // tiles whose entries are loaded at startup
constexpr int kRefillWave = 7;                  // one of the waves with the fewest gathers
constexpr int kFBW = kValue / 16 / kAttnWaves;  // 4 output feature blocks per wave
constexpr int kNHB = kHPB / 16;                 // 8 head blocks
static_assert(AttnLayout<false>::kBlocks == 36 && AttnLayout<false>::kMainBlocks == 32, "bf16");
static_assert(AttnLayout<true>::kBlocks == 18 && AttnLayout<true>::kMainBlocks == 16, "fp8");
static_assert(kSlotRing >= 2 * AttnLayout<true>::kAhead + 2 &&
              kSlotRing >= 2 * AttnLayout<false>::kAhead + 2, "slot ring holds t .. t+2*ahead+1");
static_assert(kSlotInit >= AttnLayout<true>::kRefill && kSlotInit >= AttnLayout<false>::kRefill,
              "tiles before the first refill are loaded at startup");
static_assert(AttnLayout<false>::kTilesB + 2 * kPB + kSlotRing * kTile * 4 + kHPB * 4 + 8 <=
                  160 * 1024, "LDS budget");

// fp32 pair -> packed bf16 (lo in the low half) by the hardware converter,
// round to nearest even: one instruction, where the bit-level form takes a
// dozen with a NaN branch and, unrolled over the epilogue, kilobytes of code
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// the lane index, recomputed where it is used: values derived from it are
// then rebuilt in two instructions instead of being held across the tile loop
__device__ __forceinline__ int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// F32OUT: the partial outputs are written as fp32 (a checking mode: no
// bf16 rounding between the attention and the combine), straight from the
// accumulators, 16 bytes (4 features of one head) per lane and store
template <bool FP8, bool OFF32, bool FULL, bool F32OUT>
__global__ __launch_bounds__(kAttnThreads) void sparse_mla_decode_kernel(
    const uint16_t* __restrict__ q, int rows, int heads, const uint8_t* __restrict__ cache,
    const float* __restrict__ cache_scale, int64_t num_slots, const int* __restrict__ slots,
    const int* __restrict__ counts, int k, int splits, float sm_scale,
    void* __restrict__ out_v, float* __restrict__ lse) {
  using Lay = AttnLayout<FP8>;
  constexpr int kDmaMax = Lay::kDmaMax;
  __shared__ __attribute__((aligned(16))) uint8_t s_tiles[Lay::kTilesB];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[2][kPB];
  __shared__ __attribute__((aligned(16))) int s_sring[kSlotRing * kTile];
  __shared__ float s_inv[kHPB];
  __shared__ int s_restart[2];

  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin in launch
  // order, so the G = gridDim.y * gridDim.z workgroups of a row (its parts,
  // splits and head groups, which all read the row's q) are given launch
  // indices 8 apart inside one run of 8*G: same XCD, same dispatch round
  int row, yz;
  {
    const int G = gridDim.y * gridDim.z;
    const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int b = L / (8 * G), w = L % (8 * G);
    const int nr = rows - 8 * b < 8 ? rows - 8 * b : 8;   // rows in this run
    row = 8 * b + w % nr;
    yz = w / nr;
  }
  const int part = (yz % gridDim.y) / splits;
  const int split = (yz % gridDim.y) % splits;
  const int hg = yz / gridDim.y;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = lane_id();
  const int n16 = lane & 15;      // head column of the 16x16 operands
  const int g4 = lane >> 4;       // k-group of the 16x16x32 operands
  const int h0 = hg * kHPB + wave * kHPW;
  const int head = h0 + n16;
  // FULL: every workgroup holds kHPB heads (heads a multiple of 128), so the
  // head-block guards below fold away
  const bool wave_on = FULL || h0 < heads;   // heads is a multiple of 16
  const int n_hb = FULL ? kNHB
                        : ((heads - hg * kHPB) / 16 < kNHB ? (heads - hg * kHPB) / 16 : kNHB);
  const int out_part = yz % gridDim.y;
  const int slot_lim = num_slots > 0x7fffffffLL ? 0x7fffffff : (int)num_slots;

  // ---- startup: count and the first tiles' slot entries ------------------------
  const int* my_slots = slots + ((int64_t)part * rows + row) * k;
  int cnt = counts ? counts[(int64_t)part * rows + row] : k;
  bf16x8_t qf[kQSteps];
  int sl0 = 0;
  if (splits == 1 && tid < kSlotInit * kTile) sl0 = my_slots[tid];   // k >= 512
  // q is requested next: it arrives while the slot entries are published and
  // the first gathers go out
  const uint16_t* qp = q + ((int64_t)row * heads + (wave_on ? head : 0)) * kLatent + 8 * g4;
#pragma unroll
  for (int kk = 0; kk < kQSteps; ++kk)
    qf[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u16x8_t*>(qp + 32 * kk));
  cnt = cnt < 0 ? 0 : (cnt > k ? k : cnt);
  if (num_slots <= 0) cnt = 0;
  // this split's slice of the part's token list
  const int per = ((cnt + splits - 1) / splits + kTile - 1) / kTile * kTile;
  const int t_lo = split * per < cnt ? split * per : cnt;
  const int t_hi = t_lo + per < cnt ? t_lo + per : cnt;
  const int n_tok = t_hi - t_lo;
  const int ntiles = (n_tok + kTile - 1) / kTile;
  auto load_first_slots = [&](bool have) {
    if (tid < kSlotInit * kTile) {
      int s = sl0;
      if (!have) {
        const int i = t_lo + tid;
        s = my_slots[i < k ? i : k - 1];
      }
      s_sring[tid] = s;
    }
  };
  // the first slot entries go to LDS in two separate branches, so that the
  // common one waits for its own load only and q stays in flight
  if (splits == 1) {
    if (tid < kSlotInit * kTile) s_sring[tid] = sl0;
  } else {
    load_first_slots(false);
  }

  f32x4_t o[kFBW][kNHB];
#pragma unroll
  for (int f = 0; f < kFBW; ++f)
#pragma unroll
    for (int hb = 0; hb < kNHB; ++hb) o[f][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float kv_scale = FP8 ? cache_scale[0] : 1.0f;
  const float qk_scale = sm_scale * kv_scale * kLog2e;
  float m_ref = -INFINITY, l_part = 0.f;
  if (tid < 2) s_restart[tid] = 0;
  lgkm_wait0();
  bar();   // first slot entries and flags ready

  // ---- LDS tile layout and lane-invariant byte offsets ------------------------
  // A tile is blocks of 1 KB: block 2x + h holds tokens 16h .. 16h+15 (t =
  // token % 16) x chunks 4x .. 4x+3 (16 bytes each: 8 bf16 features, or 16
  // fp8 codes).  Token t occupies slots 4t .. 4t+3, chunk 4x + c in slot 4t +
  // (c ^ rot) with rot = 2*(t/8) (bf16) or 2*(t/8) ^ h (fp8).  The chunk's
  // position is bits 4-5 of its byte offset, so another chunk of the same
  // token is an xor of the offset away.  This LDS serves a 16-byte read in
  // four passes over 16 lanes (lane bit 5 and the parity of lane bits 2-4
  // select the pass), each pass needing 16 different 16-byte bank windows
  // (address mod 256); in-bounds probes of every read pattern below time
  // them at or under the cost of contiguous reads, where other rotations
  // (by t/4, or none) doubled the score reads' cost.
  //  - bf16 scores, k-step kk, token half b: lane (n16, g4) reads chunk g4 of
  //    block 2kk + b for token n16 at qk_off + 2048*kk + 1024*b;
  //  - bf16 values: in 16-lane group g4, source lane s = n16 reads token
  //    16*rd + 4*g4 + s/4 at features 16*fb + 4*(s%4): chunk 2fb + (s%4)/2,
  //    half s%2, at (pv_off ^ 32*(fb%2)) + 2048*(fb/2) + 1024*rd;
  //  - fp8 scores, k-step kk, token half b: lane (n16, g4) reads the 8 codes
  //    of features 32kk + 8*g4 .. +8 of token 16b + n16 (chunk 2kk + g4/2,
  //    half g4%2) at (qo8_h ^ 32*(kk%2) ^ 16*b) + 2048*(kk/2) + 1024*b;
  //  - fp8 values, block fb (chunk fb): ds_read_b64_tr_b8 hands lane i of a
  //    16-lane group byte i%8 of the 8-byte chunk addressed by lane 2e + i/8
  //    of its group as element e, so lane (s, g4) addresses half s%2 of the
  //    token that element s/2 stands for (4*g4 + e%4, + 16 for e >= 4), at
  //    (po8_h ^ 16*(fb%4)) + 2048*(fb/4); lane i then holds feature i of
  //    the block for the 8 tokens in the order of the P^T operand.
  // The bf16 offsets are rebuilt from the lane index where they are used:
  // held across the tile loop they would cost spill slots.
  auto qk_off = [&]() {
    const int l = lane_now(), m = l & 15, g = l >> 4;
    return 16 * (4 * m + (g ^ (2 * (m >> 3))));
  };
  auto pv_off = [&]() {   // feature blocks of even fb; odd: xor 32
    const int l = lane_now(), m = l & 15, g = l >> 4;
    return 64 * (4 * g + (m >> 2)) + 32 * (g >> 1) + 16 * ((m >> 1) & 1) + 8 * (m & 1);
  };
  // fp8: the two offsets are held across the loop (registers are free there,
  // and the conversions leave the wave less VALU time to rebuild them)
  // scores: token half 0, even kk
  const int qo8_h = FP8 ? 64 * n16 + 16 * ((g4 >> 1) ^ (2 * (n16 >> 3))) + 8 * (g4 & 1) : 0;
  // values: chunk 4x of the block; chunk 4x + f: xor 16f
  const int po8_h = FP8 ? 1024 * ((n16 >> 1) >> 2) + 64 * (4 * g4 + ((n16 >> 1) & 3)) +
                              16 * ((2 * (g4 >> 1)) ^ ((n16 >> 1) >> 2)) + 8 * (n16 & 1) : 0;

  auto main_stage = [&](int tt) { return s_tiles + (tt % Lay::kMainStages) * Lay::kMainB; };
  auto rope_stage = [&](int tt) {
    return s_tiles + Lay::kMainStages * Lay::kMainB + (tt % Lay::kRopeStages) * Lay::kRopeB;
  };
  // this wave's vector-memory operations for tile u: its gathers, and for the
  // refill wave the copy of tile u + kRefill's slot entries
  const int my_dma = Lay::kBlocks / kAttnWaves + (wave < Lay::kBlocks % kAttnWaves ? 1 : 0);
  auto refills = [&](int u) {
    return wave == kRefillWave && u + Lay::kRefill >= kSlotInit && u + Lay::kRefill < ntiles;
  };
  // gather instruction ins fills block ins: lane l takes token 16*(ins%2) +
  // l/4 and chunk 4*(ins/2) + ((l%4) ^ rot); a wave's instructions are ins =
  // wave + 8j, so all of them cover the same 16 tokens and one slot entry per
  // lane serves the wave's whole tile
  auto tile_slot = [&](int u) {
    return s_sring[(u % kSlotRing) * kTile + 16 * (wave & 1) + (lane_now() >> 2)];
  };
  auto issue = [&](int u, int sv) {
    const int gl = lane_now();
    const int g_rot = (2 * (gl >> 5)) ^ (FP8 ? (wave & 1) : 0);
    if (refills(u) && lane < kTile) {
      const int v = u + Lay::kRefill;
      const int i = t_lo + v * kTile + lane_now();
      __builtin_amdgcn_global_load_lds((const void*)(my_slots + (i < k ? i : k - 1)),
                                       (lds_void_ptr)(s_sring + (v % kSlotRing) * kTile), 4, 0, 0);
    }
    uint8_t* ms = main_stage(u);
    uint8_t* rs = rope_stage(u);
#pragma unroll
    for (int jj = 0; jj < kDmaMax; ++jj) {
      const int ins = jj * kAttnWaves + wave;
      if (ins < Lay::kBlocks) {
        const int off = (4 * (ins >> 1) + ((gl & 3) ^ g_rot)) * 16;
        const int s = (unsigned)sv < (unsigned)slot_lim ? sv : 0;
        const uint8_t* src;
        if constexpr (OFF32)
          src = cache + (uint32_t)((uint32_t)s * (uint32_t)Lay::kRowBytes + (uint32_t)off);
        else
          src = cache + (int64_t)s * Lay::kRowBytes + off;
        uint8_t* dst = ins < Lay::kMainBlocks ? ms + ins * 1024 : rs + (ins - Lay::kMainBlocks) * 1024;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_ptr)dst, 16, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // S^T = K Q^T for token blocks 0..15 (s0) and 16..31 (s1); the key operands
  // are read kKAhead k-steps ahead of their products
  auto scores = [&](int tt, f32x4_t& s0, f32x4_t& s1) {
    s0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    s1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (!wave_on) return;
    constexpr int A = Lay::kKAhead;
    if constexpr (FP8) {
      // key offsets: half 0 even kk qo, odd qo ^ 32; half 1 even qo ^ 16,
      // odd qo ^ 48 (plus 1024)
      const int qo = qo8_h;
      const uint32_t ms = (uint32_t)(uintptr_t)(lds_void_ptr)main_stage(tt);
      const uint32_t rs = (uint32_t)(uintptr_t)(lds_void_ptr)rope_stage(tt);
      const uint32_t m00 = ms + qo, m01 = ms + (qo ^ 32), m10 = ms + (qo ^ 16), m11 = ms + (qo ^ 48);
      i32x2_t ka[kQSteps], kb[kQSteps];
      auto rd = [&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        if constexpr (kk < 16) {
          ka[kk] = lds_read_b64<2048 * (kk >> 1)>(kk & 1 ? m01 : m00);
          kb[kk] = lds_read_b64<2048 * (kk >> 1) + 1024>(kk & 1 ? m11 : m10);
        } else {
          ka[kk] = lds_read_b64<0>(rs + (kk & 1 ? (qo ^ 32) : qo));
          kb[kk] = lds_read_b64<1024>(rs + (kk & 1 ? (qo ^ 48) : (qo ^ 16)));
        }
      };
      static_for<A>([&](auto kc) { rd(kc); });
      static_for<kQSteps>([&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        constexpr int last = kk + A - 1 < kQSteps - 1 ? kk + A - 1 : kQSteps - 1;
        lgkm_wait_2v<2 * (last - kk)>(ka[kk], kb[kk]);
        if constexpr (kk + A < kQSteps) rd(IntC<kk + A>{});
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(ka[kk].x, ka[kk].y), qf[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(kb[kk].x, kb[kk].y), qf[kk], s1, 0, 0, 0);
      });
    } else {
      const int qo = qk_off();
      const uint32_t ma = (uint32_t)(uintptr_t)(lds_void_ptr)(main_stage(tt) + qo);
      const uint32_t ra = (uint32_t)(uintptr_t)(lds_void_ptr)(rope_stage(tt) + qo);
      u32x4_t ka[kQSteps], kb[kQSteps];
      auto rd = [&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        if constexpr (kk < 16) {
          ka[kk] = lds_read_b128<2048 * kk>(ma);
          kb[kk] = lds_read_b128<2048 * kk + 1024>(ma);
        } else {
          ka[kk] = lds_read_b128<2048 * (kk - 16)>(ra);
          kb[kk] = lds_read_b128<2048 * (kk - 16) + 1024>(ra);
        }
      };
      static_for<A>([&](auto kc) { rd(kc); });
      static_for<kQSteps>([&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        constexpr int last = kk + A - 1 < kQSteps - 1 ? kk + A - 1 : kQSteps - 1;
        lgkm_wait_2<2 * (last - kk)>(ka[kk], kb[kk]);
        if constexpr (kk + A < kQSteps) rd(IntC<kk + A>{});
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[kk]), qf[kk],
                                                     s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kb[kk]), qf[kk],
                                                     s1, 0, 0, 0);
      });
    }
  };
  // O^T += V^T P^T for this wave's 4 feature blocks and every present head
  // block; the P^T of head block hb is what lane `lane` of score wave hb wrote.
  // bf16: the P^T fragments go through a ring of two, read one head block
  // ahead of its products, the first two requested with the value fragments
  // (read as they are used, each read's round trip stalls the wave before
  // its 4 products: decode 62.7 -> 58.8 us).  fp8 keeps the plain reads: with
  // its conversions the ring's 4 registers cost more than the overlap gains.
  auto values = [&](int tt) {
    bf16x8_t va[kFBW];
    u32x4_t pr[2];
    uint32_t pb = 0;
    if constexpr (!FP8) pb = (uint32_t)(uintptr_t)(lds_void_ptr)(s_p[tt & 1] + 16 * lane_now());
    if constexpr (FP8) {
      // features 16*(4*wave + f) + lane%16, 8 tokens in the P^T order
      const uint32_t vb = (uint32_t)(uintptr_t)(lds_void_ptr)(main_stage(tt) + 2048 * wave);
      const int po = po8_h;
      i32x2_t r[kFBW];
      static_for<kFBW>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        r[f] = lds_read_tr8<0>(vb + (po ^ (16 * f)));
      });
      lgkm_wait_4v<0>(r[0], r[1], r[2], r[3]);
#pragma unroll
      for (int f = 0; f < kFBW; ++f) va[f] = widen8((uint32_t)r[f].x, (uint32_t)r[f].y);
    } else {
      // ds_read_b64_tr_b16 of features 16*(4*wave + f) + lane%16 for tokens
      // 4*g4 + e (first read) and 16 + 4*g4 + e (second)
      const int po = pv_off();
      const uint32_t vb0 = (uint32_t)(uintptr_t)(lds_void_ptr)(main_stage(tt) + 4096 * wave + po);
      const uint32_t vb1 =
          (uint32_t)(uintptr_t)(lds_void_ptr)(main_stage(tt) + 4096 * wave + (po ^ 32));
      i32x2_t r[2 * kFBW];
      static_for<kFBW>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        r[2 * f] = lds_read_tr16<2048 * (f >> 1)>(f & 1 ? vb1 : vb0);
        r[2 * f + 1] = lds_read_tr16<2048 * (f >> 1) + 1024>(f & 1 ? vb1 : vb0);
      });
      pr[0] = lds_read_b128<0>(pb);
      pr[1] = lds_read_b128<1024>(pb);
      lgkm_wait_4v<2>(r[0], r[1], r[2], r[3]);
      lgkm_wait_4v<2>(r[4], r[5], r[6], r[7]);
#pragma unroll
      for (int f = 0; f < kFBW; ++f)
        va[f] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r[2 * f], r[2 * f + 1], 0, 1, 2, 3));
    }
    if constexpr (FP8) {
      const uint8_t* pp = s_p[tt & 1] + 16 * lane;
      bf16x8_t pa = *reinterpret_cast<const bf16x8_t*>(pp);
#pragma unroll
      for (int hb = 0; hb < kNHB; ++hb) {
        if (hb < n_hb) {
          bf16x8_t pn = pa;
          if (hb + 1 < n_hb) pn = *reinterpret_cast<const bf16x8_t*>(pp + 1024 * (hb + 1));
#pragma unroll
          for (int f = 0; f < kFBW; ++f)
            o[f][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[f], pa, o[f][hb], 0, 0, 0);
          pa = pn;
        }
      }
    } else {
      // every head block's fragment is read (s_p holds all 8; absent blocks
      // are never used), so the ring's wait counts are fixed
      static_for<kNHB>([&](auto hc) {
        constexpr int hb = decltype(hc)::value;
        lgkm_wait_1<hb + 1 < kNHB ? 1 : 0>(pr[hb & 1]);
        if (hb < n_hb) {
          const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, pr[hb & 1]);
#pragma unroll
          for (int f = 0; f < kFBW; ++f)
            o[f][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[f], pa, o[f][hb], 0, 0, 0);
        }
        if constexpr (hb + 2 < kNHB) pr[hb & 1] = lds_read_b128<1024 * (hb + 2)>(pb);
      });
    }
  };
  // mask, softmax against the reference max, P^T of tile tt to LDS.  sv: the
  // slot entry of token lane % 32 of the tile; tokens past the tile's end are
  // masked by position
  auto finish = [&](int tt, int sv, f32x4_t s0, f32x4_t s1) {
    const int tbase = tt * kTile;
    const int ln = lane_now();
    const uint32_t vmask = (uint32_t)__ballot(ln < kTile && tbase + ln < n_tok &&
                                              (unsigned)sv < (unsigned)slot_lim);
    if (!wave_on) return;
    // lane holds head `head`, tokens 4*g4 + i (s0) and 16 + 4*g4 + i (s1)
    if (vmask != 0xffffffffu) {
      const uint32_t mv = vmask >> (4 * (lane_now() >> 4));   // bit i: token 4*g4 + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s0[i] = (mv >> i) & 1u ? s0[i] : -INFINITY;
        s1[i] = (mv >> (16 + i)) & 1u ? s1[i] : -INFINITY;
      }
    }
    float mt = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                     fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    // max over the head's four lanes (n16 + 16j): swap 16-lane rows 0<->1 and
    // 2<->3, then the two 32-lane halves; each swap returns both operands,
    // whose max is the pairwise max in every lane
    {
      const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                      false, false);
      mt = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
      const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                      false, false);
      mt = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1])) * qk_scale;
    }
    if (m_ref == -INFINITY) {
      m_ref = mt;
    } else if (__any(mt > m_ref + kRestartSlack)) {
      m_ref = fmaxf(m_ref, mt);
      if (lane == 0) s_restart[tt & 1] = 1;
    }
    const float nm = (m_ref == -INFINITY) ? 0.f : -m_ref;
    // P^T operand: element e < 4 is token 4*g4 + e, element 4 + e is token
    // 16 + 4*g4 + e (the value fragments use the same token order)
    bf16x8_t pf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], qk_scale, nm));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], qk_scale, nm));
      l_part += p0;
      l_part += p1;
      pf[i] = static_cast<__bf16>(p0);
      pf[4 + i] = static_cast<__bf16>(p1);
    }
    *reinterpret_cast<bf16x8_t*>(s_p[tt & 1] + (wave * kWave + lane_now()) * 16) = pf;
  };

  // the first kAhead tiles' slot entries are all read before a gather is issued
  auto start = [&]() {
    int sv[Lay::kAhead];
#pragma unroll
    for (int u = 0; u < Lay::kAhead; ++u) sv[u] = tile_slot(u);
#pragma unroll
    for (int u = 0; u < Lay::kAhead; ++u)
      if (u < ntiles) issue(u, sv[u]);
  };
  start();
  // everything in flight (q, the first tiles) is waited for before the loop,
  // so that inside it q is plain registers
  asm volatile("s_waitcnt vmcnt(0)"
               : "+v"(qf[0]), "+v"(qf[1]), "+v"(qf[2]), "+v"(qf[3]), "+v"(qf[4]), "+v"(qf[5]),
                 "+v"(qf[6]), "+v"(qf[7]), "+v"(qf[8]), "+v"(qf[9]), "+v"(qf[10]), "+v"(qf[11]),
                 "+v"(qf[12]), "+v"(qf[13]), "+v"(qf[14]), "+v"(qf[15]), "+v"(qf[16]),
                 "+v"(qf[17])
               :
               : "memory");
  // A restart request raised while finishing tile t goes to flag slot t % 2
  // and is read after the next barrier, in iteration t+1 (the last tile's in
  // the extra iteration t = ntiles, which only finishes the values).  With two
  // slots, a fast wave raising a request never writes the slot a slower wave
  // may still be reading.
  for (int t = 0; t <= ntiles;) {
    {   // wait for this wave's gathers of tile t: those of later tiles may fly
      int after = 0;
#pragma unroll
      for (int d = 1; d < Lay::kAhead; ++d)
        if (t + d < ntiles) after += my_dma + (refills(t + d) ? 1 : 0);
      if (t < ntiles) vm_wait_n(after);
      else vm_wait<0>();
    }
    lgkm_wait0();
    bar();   // tile t visible; P^T of tile t-1 written; every wave done with tile t-2
    const int rflag = s_restart[(t + 1) & 1];   // raised while finishing tile t-1
    const int sv = t < ntiles ? s_sring[(t % kSlotRing) * kTile + (lane & 31)] : 0;
    if (t + Lay::kAhead < ntiles) {
      issue(t + Lay::kAhead, tile_slot(t + Lay::kAhead));
    }
    // the two matrix phases run at raised wave priority: where the two waves
    // of a SIMD are in different phases, the softmax and gather issue of one
    // yield to the products of the other
    __builtin_amdgcn_s_setprio(1);
    if (t >= 1) values(t - 1);
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t s0, s1;
    if (t < ntiles) scores(t, s0, s1);
    __builtin_amdgcn_s_setprio(0);
    if (__builtin_amdgcn_readfirstlane(rflag)) {
      // a reference max moved by more than 2^64: drop the partial sums and
      // replay the token list with the raised reference
      vm_wait<0>();
      lgkm_wait0();
      bar();
      if (tid < 2) s_restart[tid] = 0;
#pragma unroll
      for (int f = 0; f < kFBW; ++f)
#pragma unroll
        for (int hb = 0; hb < kNHB; ++hb) o[f][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      l_part = 0.f;
      load_first_slots(false);
      __syncthreads();
      start();
      t = 0;
      continue;
    }
    if (t < ntiles) finish(t, sv, s0, s1);
    ++t;
  }

  // ---- epilogue ---------------------------------------------------------------
  // the lane's indexes are rebuilt here rather than held across the loop
  // (keeping them costs spill slots, and scratch costs every launch)
  const int e_lane = lane_now();
  const int e_n16 = e_lane & 15, e_g4 = e_lane >> 4;
  float l_tot = l_part + __shfl_xor(l_part, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  if (wave_on && e_g4 == 0) {
    s_inv[wave * kHPW + e_n16] = l_tot > 0.f ? kv_scale / l_tot : 0.f;
    const float lv = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
    lse[((int64_t)out_part * rows + row) * heads + h0 + e_n16] = lv;
  }
  lgkm_wait0();
  bar();   // 1/l of every head published; every wave done with the ring
  if constexpr (F32OUT) {
    // lane (n16, g4) holds features 64*wave + 16*f + 4*g4 .. +4 of head
    // 16*hb + n16 in o[f][hb]
    float* ob = reinterpret_cast<float*>(out_v) +
                (((int64_t)out_part * rows + row) * heads + hg * kHPB) * kValue;
#pragma unroll
    for (int hb = 0; hb < kNHB; ++hb) {
      if (hb < n_hb) {
        const float inv = s_inv[16 * hb + e_n16];
        float* orow = ob + (int64_t)(16 * hb + e_n16) * kValue + 64 * wave + 4 * e_g4;
#pragma unroll
        for (int f = 0; f < kFBW; ++f)
          *reinterpret_cast<float4*>(orow + 16 * f) =
              make_float4(o[f][hb][0] * inv, o[f][hb][1] * inv, o[f][hb][2] * inv,
                          o[f][hb][3] * inv);
      }
    }
    return;
  }
  uint16_t* out = reinterpret_cast<uint16_t*>(out_v);
  // staging: head rows of 512 bf16 outputs, padded by 16 bytes so that the
  // row-strided 8-byte writes spread over the banks
#pragma unroll
  for (int hb = 0; hb < kNHB; ++hb) {
    if (hb < n_hb) {
      const float inv = s_inv[16 * hb + e_n16];
      uint8_t* stg = s_tiles + (16 * hb + e_n16) * kEpiRow + (64 * wave + 4 * e_g4) * 2;
#pragma unroll
      for (int f = 0; f < kFBW; ++f) {
        const uint2 v = make_uint2(cvt_pk_bf16(o[f][hb][0] * inv, o[f][hb][1] * inv),
                                   cvt_pk_bf16(o[f][hb][2] * inv, o[f][hb][3] * inv));
        *reinterpret_cast<uint2*>(stg + 32 * f) = v;
      }
    }
  }
  lgkm_wait0();
  bar();
  if (wave_on) {
    uint16_t* ob = out + (((int64_t)out_part * rows + row) * heads + h0) * kValue;
#pragma unroll
    for (int r = 0; r < kHPW; ++r) {
      const uint4 v = *reinterpret_cast<const uint4*>(s_tiles + (wave * kHPW + r) * kEpiRow + e_lane * 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(ob + (int64_t)r * kValue) + e_lane * 16) = v;
    }
  }
}

int launch_sparse_mla_decode(const void* q, int rows, int heads, const void* cache, bool fp8,
                             const float* cache_scale, int64_t num_slots, const int* slots,
                             const int* counts, int k, int n_parts, int splits, float sm_scale,
                             void* out, bool f32out, float* lse, hipStream_t stream) {
  dim3 grid(rows, n_parts * splits, (heads + kHPB - 1) / kHPB);
  const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q);
  const uint8_t* c8 = reinterpret_cast<const uint8_t*>(cache);
  // 32-bit gather offsets when the whole pool lies within 4 GiB of its base
  const bool off32 = num_slots * (int64_t)(fp8 ? kRowB8 : kRowB) <= (int64_t)0xffffffffLL;
  const bool full = heads % kHPB == 0;
  // fp32 partials (the checking mode) take the general head-group variant
#define DSA_ATTN(F, O)                                                                       \
  if (f32out)                                                                                \
    hipLaunchKernelGGL((sparse_mla_decode_kernel<F, O, false, true>), grid, dim3(kAttnThreads), \
                       0, stream, q16, rows, heads, c8, cache_scale, num_slots, slots, counts, \
                       k, splits, sm_scale, out, lse);                                        \
  else if (full)                                                                             \
    hipLaunchKernelGGL((sparse_mla_decode_kernel<F, O, true, false>), grid, dim3(kAttnThreads), \
                       0, stream, q16, rows, heads, c8, cache_scale, num_slots, slots, counts, \
                       k, splits, sm_scale, out, lse);                                        \
  else                                                                                       \
    hipLaunchKernelGGL((sparse_mla_decode_kernel<F, O, false, false>), grid, dim3(kAttnThreads), \
                       0, stream, q16, rows, heads, c8, cache_scale, num_slots, slots, counts, \
                       k, splits, sm_scale, out, lse)
  if (fp8) {
    if (off32) { DSA_ATTN(true, true); }
    else { DSA_ATTN(true, false); }
  } else {
    if (off32) { DSA_ATTN(false, true); }
    else { DSA_ATTN(false, false); }
  }
#undef DSA_ATTN
  return 0;
}

}  // namespace dsa
