// route_topk.hip -- top-k expert selection and softmax gate weights.
//
// Strata feature (tech.hub77a.com), summary row "핵심 기법" and section
// "2. 왜 대단한가" (1)-(2): the router picks a few experts per token and only
// those run.  Selection: the k largest logits, descending, equal logits rank
// the lower expert id first, -0.0 equals +0.0.  Weights: softmax over the k
// selected logits.
//
// One wave64 per token (the per-token routine is shared with the decode-step
// kernels, so all produce identical bits).  Each lane owns E/64 logits
// (lane-strided, so the row is read with coalesced loads).  A logit becomes a
// 32-bit key whose unsigned order is the float order (sign-magnitude to offset
// binary; +0 and -0 share one key), so the selection is exact integer work: a
// threshold from the lane maxima narrows the row to a few candidates, which
// rank themselves in (key descending, id ascending) order.
#include "route_dispatch_dev.hpp"

namespace moe {
namespace {

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ dev::TopkLds S[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int id;
  float wt;
  dev::route_token<EPL>(logits + (size_t)t * E, E, k, id, wt, S[wave]);
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
