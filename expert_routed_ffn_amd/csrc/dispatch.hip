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
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kBlock = 1024;
constexpr int kWaves = kBlock / 64;
constexpr int kSmallN = 4096;
constexpr int kSentinel = 2047;  // 11 bits; never a valid id (E <= 1024)

__device__ __forceinline__ uint64_t match_peers(int key) {
  uint64_t peers = ~0ull;
#pragma unroll
  for (int b = 0; b < 11; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// Exclusive scan over the block of two values at once; returns the totals.
__device__ __forceinline__ void block_exclusive_scan2(int v0, int v1, int& ex0, int& ex1, int& tot0, int& tot1,
                                                      int* sh /* [2 * kWaves] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int s0 = v0, s1 = v1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a0 = __shfl_up(s0, off, 64), a1 = __shfl_up(s1, off, 64);
    if (lane >= off) { s0 += a0; s1 += a1; }
  }
  if (lane == 63) { sh[wave] = s0; sh[kWaves + wave] = s1; }
  __syncthreads();
  int b0 = 0, b1 = 0, t0 = 0, t1 = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int c0 = sh[w], c1 = sh[kWaves + w];
    if (w < wave) { b0 += c0; b1 += c1; }
    t0 += c0;
    t1 += c1;
  }
  ex0 = b0 + s0 - v0;
  ex1 = b1 + s1 - v1;
  tot0 = t0;
  tot1 = t1;
  __syncthreads();
}

// Counts -> offsets, cursor (LDS copy of offsets), active list, n_active.
__device__ __forceinline__ void offsets_and_active(const int* cnt_lds, int E, int32_t* offsets, int* cursor,
                                                   int32_t* active, int32_t* n_active, int* scan_sh) {
  const int tid = threadIdx.x;
  const int c = tid < E ? cnt_lds[tid] : 0;
  int exc, exf, totc, totf;
  block_exclusive_scan2(c, c > 0 ? 1 : 0, exc, exf, totc, totf, scan_sh);
  if (tid < E) {
    offsets[tid] = exc;
    if (cursor) cursor[tid] = exc;
    if (c > 0) active[exf] = tid;
  }
  if (tid == 0) {
    offsets[E] = totc;
    *n_active = totf;
  }
}

__global__ __launch_bounds__(kBlock) void dispatch_small_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted_assign,
                                                                int32_t* __restrict__ assign_pos,
                                                                int32_t* __restrict__ active,
                                                                int32_t* __restrict__ n_active) {
  __shared__ int cnt[kMaxE];
  __shared__ int cursor[kMaxE];
  __shared__ int scan_sh[2 * kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  for (int a = tid; a < n; a += kBlock) {
    const int e = ids[a];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  offsets_and_active(cnt, E, offsets, cursor, active, n_active, scan_sh);
  __syncthreads();

  const uint64_t lt = (1ull << lane) - 1ull;
  for (int base = 0; base < n; base += kBlock) {
    const int a = base + tid;
    const bool valid = a < n;
    const int e = valid ? ids[a] : -1;
    const bool ok = valid && (unsigned)e < (unsigned)E;
    const uint64_t peers = match_peers(ok ? e : kSentinel);
    const int rank = __popcll(peers & lt), cnt_w = __popcll(peers);
    const int nw = (int)min((int64_t)kWaves, ceil_div(n - base, 64));
    for (int w = 0; w < nw; ++w) {
      if (wave == w && ok) {
        const int pos = cursor[e] + rank;
        sorted_assign[pos] = a;
        assign_pos[a] = pos;
        if (rank == cnt_w - 1) cursor[e] = pos + 1;
      }
      __syncthreads();
    }
    if (valid && !ok) assign_pos[a] = -1;
  }
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
  const uint64_t peers = match_peers(ok ? e : kSentinel);
  const uint64_t lt = (1ull << lane) - 1ull;
  const int rank = __popcll(peers & lt), cnt_w = __popcll(peers);
  const int nw = (int)min((int64_t)kWaves, ceil_div(n - base, 64));
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
  __shared__ int scan_sh[2 * kWaves];
  const int tid = threadIdx.x;
  if (tid < E) {
    int run = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int v = chunk_count[(size_t)c * E + tid];
      chunk_count[(size_t)c * E + tid] = run;
      run += v;
    }
    cnt[tid] = run;
  }
  __syncthreads();
  offsets_and_active(cnt, E, offsets, nullptr, active, n_active, scan_sh);
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
