// LSE-weighted combine of per-shard partial attention outputs.
//
// What is computed (PR #52046 report, 关键源码片段: `dcp_manager.combine(
// attn_out, lse, ...)` merges the shards' partials; PR #46076 report,
// 评论区精华: the reducer works in base e):
//   lse = ln sum_p exp(lse_p) over finite lse_p, out = sum_p exp(lse_p - lse) out_p.
// A (row, head) whose partials are all empty gets out = 0, lse = -inf.
//
// How: a pure streaming kernel — one thread per (row, head, 8 features),
// fp32 accumulation in partial order, 16-byte bf16 store.  With at most 8
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
// fp32 pair -> packed bf16 (lo in the low half), hardware round to nearest even
__device__ __forceinline__ uint32_t cvt_pk_bf16c(float lo, float hi) {
  typedef __bf16 bf16x2c_t __attribute__((ext_vector_type(2)));
  const bf16x2c_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// NF > 0: up to NF partials, all loads in flight at once; NF == 0: any number
template <int NF>
__global__ __launch_bounds__(kCombineThreads) void lse_combine_kernel(
    const uint16_t* __restrict__ pout, const float* __restrict__ plse, int P, int64_t rh_total,
    int dim, uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  const int chunks = dim / 8;
  const int64_t gid = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  if (gid >= rh_total * chunks) return;
  const int64_t rh = gid / chunks;
  const int c = (int)(gid % chunks);
  auto slice = [&](int p) {
    return reinterpret_cast<const uint4*>(pout + ((int64_t)p * rh_total + rh) * dim + c * 8);
  };

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float z = 0.f, M = -INFINITY;
  if constexpr (NF > 0) {
    float l[NF];
    uint4 v[NF];
#pragma unroll
    for (int p = 0; p < NF; ++p) {
      l[p] = -INFINITY;
      v[p] = make_uint4(0u, 0u, 0u, 0u);
      if (p < P) {
        l[p] = plse[(int64_t)p * rh_total + rh];
        v[p] = *slice(p);
      }
    }
#pragma unroll
    for (int p = 0; p < NF; ++p) M = fmaxf(M, l[p]);
    if (M != -INFINITY) {
#pragma unroll
      for (int p = 0; p < NF; ++p) {
        const float w = exp2f((l[p] - M) * kLog2eC);   // exp(-inf) = 0
        z += w;
        accumulate8(acc, w, v[p]);
      }
    }
  } else {
    for (int p = 0; p < P; ++p) M = fmaxf(M, plse[(int64_t)p * rh_total + rh]);
    if (M != -INFINITY) {
      constexpr int B = 4;
      for (int p0 = 0; p0 < P; p0 += B) {
        uint4 v[B];
        float w[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int p = p0 + b;
          w[b] = 0.f;
          v[b] = make_uint4(0u, 0u, 0u, 0u);
          if (p < P) {
            w[b] = exp2f((plse[(int64_t)p * rh_total + rh] - M) * kLog2eC);
            v[b] = *slice(p);
          }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          z += w[b];
          accumulate8(acc, w[b], v[b]);
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

int launch_lse_combine(const void* part_out, const float* part_lse, int P, int rows, int heads,
                       int dim, void* out, float* lse_out, hipStream_t stream) {
  const int64_t rh = (int64_t)rows * heads;
  const int64_t threads = rh * (dim / 8);
  const int64_t blocks = (threads + kCombineThreads - 1) / kCombineThreads;
  const uint16_t* po = reinterpret_cast<const uint16_t*>(part_out);
  uint16_t* o = reinterpret_cast<uint16_t*>(out);
  if (P <= 8)
    hipLaunchKernelGGL(lse_combine_kernel<8>, dim3((unsigned)blocks), dim3(kCombineThreads), 0,
                       stream, po, part_lse, P, rh, dim, o, lse_out);
  else if (P <= kCombineFast)
    hipLaunchKernelGGL(lse_combine_kernel<kCombineFast>, dim3((unsigned)blocks),
                       dim3(kCombineThreads), 0, stream, po, part_lse, P, rh, dim, o, lse_out);
  else
    hipLaunchKernelGGL(lse_combine_kernel<0>, dim3((unsigned)blocks), dim3(kCombineThreads), 0,
                       stream, po, part_lse, P, rh, dim, o, lse_out);
  return 0;
}

}  // namespace dsa
