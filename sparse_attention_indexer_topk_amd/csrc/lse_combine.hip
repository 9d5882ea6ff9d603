// LSE-weighted combine of per-shard partial attention outputs.
//
// What is computed (PR #52046 report, 关键源码片段: `dcp_manager.combine(
// attn_out, lse, ...)` merges the shards' partials; PR #46076 report,
// 评论区精华: the reducer works in base e):
//   lse = ln sum_p exp(lse_p) over finite lse_p, out = sum_p exp(lse_p - lse) out_p.
// A (row, head) whose partials are all empty gets out = 0, lse = -inf.
//
// How: a pure streaming kernel — one thread per (row, head) and one 8-feature
// slice, or two slices half a row apart for small launches, fp32
// accumulation in partial order, 16-byte bf16 stores.  Two slices per thread
// keep twice the bytes in flight per wave where the launch is too small to
// fill the memory system with threads (at most 8 partials and 64K (row,
// head) pairs: decode 8.6 -> 7.8 us, fp8 15.5 -> 14.4 us); with more
// partials, or a launch as large as a prefill chunk, they were slower.  The partials are
// bf16 (the path's format) or fp32 (the attention's checking mode), read as
// one 16-byte or two 16-byte slices per partial.  With at most 8
// or 16 partials every load (the partial LSEs and the 16-byte output slices)
// is issued before the first is used, so a thread makes one memory round
// trip; more partials are taken four at a time.
#include "launchers.h"

namespace dsa {

constexpr int kCombineThreads = 256;
constexpr int kCombineFast = 16;  // most partials held in registers at once
constexpr float kLog2eC = 1.4426950408889634f;

// acc += w * v for the 8 bf16 values of v; a zero weight (an empty partial,
// or a slot past the partial count) adds nothing, whatever v holds
__device__ __forceinline__ void accumulate8(float (&acc)[8], float w, const uint4 v) {
  const bool on = w != 0.f;
  const uint32_t ws[4] = {on ? v.x : 0u, on ? v.y : 0u, on ? v.z : 0u, on ? v.w : 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] += w * bf16_to_f32((uint16_t)(ws[e >> 1] >> (16 * (e & 1))));
}
// the same for 8 fp32 values
__device__ __forceinline__ void accumulate8(float (&acc)[8], float w, const float4 a,
                                            const float4 b) {
  const bool on = w != 0.f;
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] += w * (on ? x[e] : 0.f);
}
// 8 partial values of one (row, head) as held in registers
template <bool F32>
struct Slice8;
template <>
struct Slice8<false> {
  uint4 v;
  __device__ __forceinline__ void zero() { v = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void add_to(float (&acc)[8], float w) const { accumulate8(acc, w, v); }
};
template <>
struct Slice8<true> {
  float4 a, b;
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void load(const void* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void add_to(float (&acc)[8], float w) const {
    accumulate8(acc, w, a, b);
  }
};

// fp32 pair -> packed bf16 (lo in the low half), hardware round to nearest even
__device__ __forceinline__ uint32_t cvt_pk_bf16c(float lo, float hi) {
  typedef __bf16 bf16x2c_t __attribute__((ext_vector_type(2)));
  const bf16x2c_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// One (row, head), features 8c .. 8c + 7.  NF > 0: up to NF partials, all
// loads in flight at once; NF == 0: any number.  F32: fp32 partials.
template <int NF, bool F32>
__device__ __forceinline__ void combine_slice(const void* __restrict__ pout,
                                              const float* __restrict__ plse, int P,
                                              int64_t rh_total, int dim, int64_t rh, int c,
                                              uint16_t* __restrict__ out,
                                              float* __restrict__ lse_out) {
  constexpr int kElem = F32 ? 4 : 2;   // bytes per partial value
  auto slice = [&](int p) {
    return reinterpret_cast<const uint8_t*>(pout) +
           (((int64_t)p * rh_total + rh) * dim + c * 8) * kElem;
  };

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float z = 0.f, M = -INFINITY;
  if constexpr (NF > 0) {
    float l[NF];
    Slice8<F32> v[NF];
#pragma unroll
    for (int p = 0; p < NF; ++p) {
      l[p] = -INFINITY;
      v[p].zero();
      if (p < P) {
        l[p] = plse[(int64_t)p * rh_total + rh];
        v[p].load(slice(p));
      }
    }
#pragma unroll
    for (int p = 0; p < NF; ++p) M = fmaxf(M, l[p]);
    if (M != -INFINITY) {
#pragma unroll
      for (int p = 0; p < NF; ++p) {
        const float w = exp2f((l[p] - M) * kLog2eC);   // exp(-inf) = 0
        z += w;
        v[p].add_to(acc, w);
      }
    }
  } else {
    for (int p = 0; p < P; ++p) M = fmaxf(M, plse[(int64_t)p * rh_total + rh]);
    if (M != -INFINITY) {
      constexpr int B = 4;
      for (int p0 = 0; p0 < P; p0 += B) {
        Slice8<F32> v[B];
        float w[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int p = p0 + b;
          w[b] = 0.f;
          v[b].zero();
          if (p < P) {
            w[b] = exp2f((plse[(int64_t)p * rh_total + rh] - M) * kLog2eC);
            v[b].load(slice(p));
          }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          z += w[b];
          v[b].add_to(acc, w[b]);
        }
      }
    }
  }
  const float inv = z > 0.f ? 1.0f / z : 0.f;
  const uint4 o = make_uint4(cvt_pk_bf16c(acc[0] * inv, acc[1] * inv),
                             cvt_pk_bf16c(acc[2] * inv, acc[3] * inv),
                             cvt_pk_bf16c(acc[4] * inv, acc[5] * inv),
                             cvt_pk_bf16c(acc[6] * inv, acc[7] * inv));
  *reinterpret_cast<uint4*>(out + rh * dim + c * 8) = o;
  if (lse_out && c == 0) lse_out[rh] = (M == -INFINITY) ? -INFINITY : M + logf(z);
}

// NC slices per thread: slice c and c + chunks/NC of one (row, head)
template <int NF, bool F32, int NC>
__global__ __launch_bounds__(kCombineThreads) void lse_combine_kernel(
    const void* __restrict__ pout, const float* __restrict__ plse, int P, int64_t rh_total,
    int dim, uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  const int per = dim / 8 / NC;
  const int64_t gid = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  if (gid >= rh_total * per) return;
  const int64_t rh = gid / per;
  const int c = (int)(gid % per);
#pragma unroll
  for (int j = 0; j < NC; ++j)
    combine_slice<NF, F32>(pout, plse, P, rh_total, dim, rh, c + j * per, out, lse_out);
}

int launch_lse_combine(const void* part_out, bool f32in, const float* part_lse, int P, int rows,
                       int heads, int dim, void* out, float* lse_out, hipStream_t stream) {
  const int64_t rh = (int64_t)rows * heads;
  const int nc = ((dim / 8) % 2 == 0 && P <= 8 && rh <= 65536) ? 2 : 1;
  const int64_t threads = rh * (dim / 8 / nc);
  const int64_t blocks = (threads + kCombineThreads - 1) / kCombineThreads;
  uint16_t* o = reinterpret_cast<uint16_t*>(out);
#define DSA_COMBINE(NF, F32)                                                                  \
  do {                                                                                        \
    if (nc == 2)                                                                              \
      hipLaunchKernelGGL((lse_combine_kernel<NF, F32, 2>), dim3((unsigned)blocks),             \
                         dim3(kCombineThreads), 0, stream, part_out, part_lse, P, rh, dim, o,  \
                         lse_out);                                                            \
    else                                                                                      \
      hipLaunchKernelGGL((lse_combine_kernel<NF, F32, 1>), dim3((unsigned)blocks),             \
                         dim3(kCombineThreads), 0, stream, part_out, part_lse, P, rh, dim, o,  \
                         lse_out);                                                            \
  } while (0)
  if (f32in) {
    if (P <= 8) DSA_COMBINE(8, true);
    else if (P <= kCombineFast) DSA_COMBINE(kCombineFast, true);
    else DSA_COMBINE(0, true);
  } else {
    if (P <= 8) DSA_COMBINE(8, false);
    else if (P <= kCombineFast) DSA_COMBINE(kCombineFast, false);
    else DSA_COMBINE(0, false);
  }
#undef DSA_COMBINE
  return 0;
}

}  // namespace dsa
