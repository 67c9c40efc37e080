// route_topk.hip -- top-k expert selection and softmax gate weights.
//
// Strata feature (tech.hub77a.com), summary row "핵심 기법" and section
// "2. 왜 대단한가" (1)-(2): the router picks a few experts per token and only
// those run.  Selection: the k largest logits, descending, equal logits rank
// the lower expert id first, -0.0 equals +0.0.  Weights: softmax over the k
// selected logits.
//
// One wave64 per token (the per-token routine is shared with the fused decode
// step).  Each lane owns E/64 logits (lane-strided, so the row is read with
// coalesced loads).  A logit becomes a 64-bit key whose order is the ranking
// order: the high word maps the float to an unsigned integer that sorts like
// the float (sign-magnitude to offset binary; +0 and -0 share one key), the
// low word is ~id so that a lower id wins a tie.  Keys are unique, so k rounds
// of "lane max, then wave max, owner drops it" give the top k exactly, with no
// floating-point comparisons.
#include "route_dispatch_dev.hpp"

namespace moe {
namespace {

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int id;
  float wt;
  dev::route_token<EPL>(logits + (size_t)t * E, E, k, id, wt);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    w[(size_t)t * k + lane] = wt;
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
