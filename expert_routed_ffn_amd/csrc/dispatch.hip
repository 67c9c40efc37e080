// dispatch.hip -- stable grouping of the T*k assignments by expert.
//
// The tokens routed to one expert are computed together (Strata feature,
// tech.hub77a.com, section "2. 왜 대단한가" (2): the compute path follows the
// routing result).  The order is made unique so results are reproducible:
// ascending expert, and ascending assignment index a = t*k + j inside one
// expert.  It is a stable counting sort:
//   - expert counts, their exclusive prefix sum (offsets) and the list of
//     experts with a nonzero count (active);
//   - the rank of each assignment among earlier assignments of its expert.
// Ranks inside a wave come from a ballot "match" on the id bits (lanes with
// the same id, popcount of the lower ones); across waves of a chunk the waves
// take turns advancing a per-expert cursor in LDS, so no step depends on the
// order in which atomics land.
//
// n <= kSmallN: one workgroup does everything in one launch (the decode case).
// Larger n: (A) per 1024-assignment chunk, ranks within the chunk and the
// chunk's per-expert counts; (B) one workgroup turns counts into per-chunk
// bases and offsets; (C) scatter.
#include <algorithm>

#include "route_dispatch_dev.hpp"
#include "slot_dev.hpp"

namespace moe {
namespace {

using dev::kDispBlock;
using dev::kDispWaves;
using dev::kSentinel;
constexpr int kBlock = kDispBlock;
constexpr int kSmallN = 4096;

__global__ __launch_bounds__(kBlock) void dispatch_small_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted_assign,
                                                                int32_t* __restrict__ assign_pos,
                                                                int32_t* __restrict__ active,
                                                                int32_t* __restrict__ n_active) {
  __shared__ dev::DispatchLds L;
  dev::dispatch_block(ids, n, E, offsets, sorted_assign, assign_pos, active, n_active, L);
}

// (A) ranks inside each 1024-assignment chunk and the chunk's counts per expert.
__global__ __launch_bounds__(kBlock) void dispatch_rank_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                               int32_t* __restrict__ rank_in_chunk,
                                                               int32_t* __restrict__ chunk_count) {
  __shared__ int cursor[kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = blockIdx.x * kBlock;
  if (tid < E) cursor[tid] = 0;
  __syncthreads();
  const int a = base + tid;
  const bool valid = a < n;
  const int e = valid ? ids[a] : -1;
  const bool ok = valid && (unsigned)e < (unsigned)E;
  const uint64_t peers = dev::match_peers(ok ? e : kSentinel);
  const uint64_t lt = (1ull << lane) - 1ull;
  const int rank = __popcll(peers & lt), cnt_w = __popcll(peers);
  const int nw = (int)min((int64_t)kDispWaves, ceil_div(n - base, 64));
  for (int w = 0; w < nw; ++w) {
    if (wave == w && ok) {
      const int r = cursor[e] + rank;
      rank_in_chunk[a] = r;
      if (rank == cnt_w - 1) cursor[e] = r + 1;
    }
    __syncthreads();
  }
  if (tid < E) chunk_count[(size_t)blockIdx.x * E + tid] = cursor[tid];
}

// (B) per-chunk bases (in place over chunk_count), offsets and the active list.
__global__ __launch_bounds__(kBlock) void dispatch_scan_kernel(int nchunks, int E, int32_t* __restrict__ chunk_count,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ active,
                                                               int32_t* __restrict__ n_active) {
  __shared__ int cnt[kMaxE];
  __shared__ int scan_sh[2 * kDispWaves];
  const int tid = threadIdx.x;
  if (tid < E) {
    // exclusive scan of this expert's per-chunk counts, 16 chunks per batch:
    // a batch's loads are issued before its stores, so they overlap instead of
    // waiting one L2 round trip each behind the previous store
    constexpr int kBatch = 16;
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = c0 + u < nchunks ? chunk_count[(size_t)(c0 + u) * E + tid] : 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (c0 + u < nchunks) {
          chunk_count[(size_t)(c0 + u) * E + tid] = run;
          run += v[u];
        }
    }
    cnt[tid] = run;
  }
  __syncthreads();
  dev::offsets_and_active(cnt, E, offsets, nullptr, active, n_active, scan_sh);
}

// (C) scatter to the sorted positions.
__global__ __launch_bounds__(kBlock) void dispatch_scatter_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                                  const int32_t* __restrict__ rank_in_chunk,
                                                                  const int32_t* __restrict__ chunk_base,
                                                                  const int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ sorted_assign,
                                                                  int32_t* __restrict__ assign_pos) {
  const int a = blockIdx.x * kBlock + threadIdx.x;
  if (a >= n) return;
  const int e = ids[a];
  if ((unsigned)e >= (unsigned)E) {
    assign_pos[a] = -1;
    return;
  }
  const int pos = offsets[e] + chunk_base[(size_t)blockIdx.x * E + e] + rank_in_chunk[a];
  sorted_assign[pos] = a;
  assign_pos[a] = pos;
}

// Decode step, part 1: the decode router (routing, grouping, descriptors) in
// one workgroup.
template <int EPL>
__global__ __launch_bounds__(kBlock) void route_dispatch_decode_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_assign, int32_t* __restrict__ assign_pos,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, SlotDesc* __restrict__ desc, int max_active,
    int32_t* __restrict__ rows, int32_t* __restrict__ nrows) {
  __shared__ dev::RouterLds L;
  dev::decode_route_lds<EPL, kBlock>(logits, T, E, k, L);
  dev::decode_route_write<kBlock>(L, T, E, k, ids, w, offsets, sorted_assign, assign_pos, active, n_active, desc,
                                  max_active, rows, nrows);
}

// Decode router, then the slot table's resolve of the routed experts, in the
// same workgroup (the active list is still in LDS).
template <int EPL>
__global__ __launch_bounds__(kBlock) void route_dispatch_resolve_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_assign, int32_t* __restrict__ assign_pos,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, SlotDesc* __restrict__ desc, int max_active,
    int32_t* __restrict__ rows, int32_t* __restrict__ nrows, SlotDevArgs sa, int layer) {
  __shared__ dev::RouterLds L;
  __shared__ dev::SlotLds<kBlock> S;
  dev::decode_route_lds<EPL, kBlock>(logits, T, E, k, L);
  dev::decode_route_write<kBlock>(L, T, E, k, ids, w, offsets, sorted_assign, assign_pos, active, n_active, desc,
                                  max_active, rows, nrows);
  dev::slot_resolve_block<kBlock>(sa, layer, L.slot_e, L.na, S);
}

__global__ void dispatch_empty_kernel(int E, int32_t* offsets, int32_t* n_active) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = 0;
  if (threadIdx.x == 0) *n_active = 0;
}

}  // namespace

size_t dispatch_ws_bytes(int n, int E) {
  if (n <= kSmallN) return 0;
  const int64_t nchunks = ceil_div(n, kBlock);
  return (size_t)(((int64_t)n + nchunks * E) * 4 + 256);
}

moe_status launch_route_dispatch_decode(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                                        int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos,
                                        int32_t* active, int32_t* n_active, const DecodeWs& W, hipStream_t s) {
  const int epl = (int)ceil_div(E, 64);
  const auto kern = epl <= 1   ? route_dispatch_decode_kernel<1>
                    : epl <= 2 ? route_dispatch_decode_kernel<2>
                    : epl <= 4 ? route_dispatch_decode_kernel<4>
                    : epl <= 8 ? route_dispatch_decode_kernel<8>
                               : route_dispatch_decode_kernel<16>;
  if (T * k > dev::kDecodeMaxN) return fail(MOE_EUNSUPPORTED, "route_dispatch_decode: T*k above 192");
  launch_k(MOE_KERNEL_ROUTE, kern, dim3(1), dim3(kBlock), 0, s, logits, T, E, k, ids, w, offsets, sorted_assign,
           assign_pos, active, n_active, W.desc, std::min(E, T * k), W.rows, W.nrows);
  return check_launch("route_dispatch_decode");
}

moe_status launch_route_dispatch_resolve(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                                         int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos,
                                         int32_t* active, int32_t* n_active, const DecodeWs& W,
                                         const moe_slot_table* t, int layer, hipStream_t s) {
  const int epl = (int)ceil_div(E, 64);
  const auto kern = epl <= 1   ? route_dispatch_resolve_kernel<1>
                    : epl <= 2 ? route_dispatch_resolve_kernel<2>
                    : epl <= 4 ? route_dispatch_resolve_kernel<4>
                    : epl <= 8 ? route_dispatch_resolve_kernel<8>
                               : route_dispatch_resolve_kernel<16>;
  if (T * k > dev::kDecodeMaxN) return fail(MOE_EUNSUPPORTED, "route_dispatch_resolve: T*k above 192");
  launch_k(MOE_KERNEL_ROUTE, kern, dim3(1), dim3(kBlock), 0, s, logits, T, E, k, ids, w, offsets, sorted_assign,
           assign_pos, active, n_active, W.desc, std::min(E, T * k), W.rows, W.nrows, slot_dev_args(t), layer);
  return check_launch("route_dispatch_resolve");
}

moe_status launch_dispatch(const int32_t* ids, int n, int E, int32_t* offsets, int32_t* sorted_assign,
                           int32_t* assign_pos, int32_t* active, int32_t* n_active, void* ws, hipStream_t s) {
  if (n == 0) {
    launch_k(MOE_KERNEL_DISPATCH, dispatch_empty_kernel, dim3(1), dim3(256), 0, s, E, offsets, n_active);
    return check_launch("dispatch_empty");
  }
  if (n <= kSmallN) {
    launch_k(MOE_KERNEL_DISPATCH, dispatch_small_kernel, dim3(1), dim3(kBlock), 0, s, ids, n, E, offsets,
             sorted_assign, assign_pos, active, n_active);
    return check_launch("dispatch_small");
  }
  const int nchunks = (int)ceil_div(n, kBlock);
  int32_t* rank = (int32_t*)ws;
  int32_t* chunk = rank + ((n + 63) / 64) * 64;
  launch_k(MOE_KERNEL_DISPATCH, dispatch_rank_kernel, dim3(nchunks), dim3(kBlock), 0, s, ids, n, E, rank, chunk);
  if (moe_status st = check_launch("dispatch_rank")) return st;
  dispatch_scan_kernel<<<1, kBlock, 0, s>>>(nchunks, E, chunk, offsets, active, n_active);
  if (moe_status st = check_launch("dispatch_scan")) return st;
  dispatch_scatter_kernel<<<nchunks, kBlock, 0, s>>>(ids, n, E, rank, chunk, offsets, sorted_assign, assign_pos);
  return check_launch("dispatch_scatter");
}

}  // namespace moe
