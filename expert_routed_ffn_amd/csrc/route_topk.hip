// route_topk.hip -- top-k expert selection and softmax gate weights.
//
// Strata feature (tech.hub77a.com), summary row "핵심 기법" and section
// "2. 왜 대단한가" (1)-(2): the router picks a few experts per token and only
// those run.  Selection: the k largest logits, descending, equal logits rank
// the lower expert id first, -0.0 equals +0.0.  Weights: softmax over the k
// selected logits.
//
// One wave64 per token.  Each lane owns E/64 logits (lane-strided, so the row
// is read with coalesced loads).  A logit becomes a 64-bit key whose order is
// the ranking order: the high word maps the float to an unsigned integer that
// sorts like the float (sign-magnitude to offset binary; +0 and -0 share one
// key), the low word is ~id so that a lower id wins a tie.  Keys are unique,
// so k rounds of "lane max, then wave max, owner drops it" give the top k
// exactly, with no floating-point comparisons.
#include "internal.hpp"

namespace moe {
namespace {

__device__ __forceinline__ uint64_t rank_key(float f, int e) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;  // -0.0 -> +0.0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;

  uint64_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    key[j] = (e < E) ? rank_key(row[e], e) : 0ull;  // 0 is below every real key
  }

  uint64_t mine = 0;  // lane j < k ends up holding the j-th selected key
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (key[j] == best) key[j] = 0;
    if (lane == r) mine = best;
  }

  const float lj = key_logit(mine);
  const float l0 = __shfl(lj, 0, 64);
  const float ex = (lane < k) ? expf(lj - l0) : 0.0f;
  const float den = wave_sum_f32(ex);
  if (lane < k) {
    ids[(size_t)t * k + lane] = (int32_t)(~(uint32_t)mine);
    w[(size_t)t * k + lane] = ex / den;
  }
}

}  // namespace

moe_status launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(T, 4)), block(256);
  const int epl = (int)ceil_div(E, 64);
  const auto kern = epl <= 1   ? route_topk_kernel<1>
                    : epl <= 2 ? route_topk_kernel<2>
                    : epl <= 4 ? route_topk_kernel<4>
                    : epl <= 8 ? route_topk_kernel<8>
                               : route_topk_kernel<16>;
  launch_k(MOE_KERNEL_ROUTE, kern, grid, block, 0, s, logits, T, E, k, ids, w);
  return check_launch("route_topk");
}

}  // namespace moe
