// route_dispatch_dev.hpp -- device functions of routing and dispatch, shared by
// the stand-alone kernels and the fused decode-step kernel so that both
// produce identical bits.
//
// Routing (Strata feature, tech.hub77a.com, summary row "핵심 기법" and
// section "2. 왜 대단한가" (1)-(2)): per token the k largest logits, descending,
// ties to the lower expert id, -0.0 == +0.0; weights = softmax over the k.
// Each logit becomes a 32-bit key whose integer order is the float order
// (offset binary), so the selection is exact integer work.  A wave owns one
// token; k rounds of "lane max, wave max, lowest id holding it" find the
// experts, all in registers.
//
// Dispatch (section "2. 왜 대단한가" (2): the compute path follows the
// routing): a stable counting sort of the assignments by expert.
#pragma once

#include "internal.hpp"

namespace moe {
namespace dev {

// Order key of a logit: integer order equals the float order, -0.0 == +0.0,
// and 0 lies below every finite logit (used for "taken" and "no expert").
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;  // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t ord) {
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  return __uint_as_float(u);
}

typedef unsigned int u32x2_dev_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Maximum over the 64 lanes, uniform: DPP inside each 16-lane row (quad
// swaps, half-row and row mirrors), then the permlane16 / permlane32 swaps
// across rows.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp32<0x141>(v));  // row_half_mirror
  v = max(v, dpp32<0x140>(v));  // row_mirror
  const u32x2_dev_t a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(a.x, a.y);
  const u32x2_dev_t b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max(b.x, b.y);
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// One token's routing by one wave.  Lane j < k returns the j-th selected id
// in *id and its weight in *wt; other lanes return id = -1.  Expert e sits in
// lane e % 64, slot e / 64.  Each round takes the wave maximum of the keys,
// then the lowest expert id holding it (the smallest slot with a match, then
// the lowest lane: ballots over the slots), and clears that one key.
template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int& id, float& wt) {
  const int lane = threadIdx.x & 63;
  // all loads first (clamped index, no branch around them), then the keys
  float lv[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) lv[j] = row[min(lane + 64 * j, E - 1)];
  uint32_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) key[j] = (lane + 64 * j < E) ? order_key(lv[j]) : 0u;
  uint32_t mine = 0;
  int mine_id = -1;
  for (int r = 0; r < k; ++r) {
    uint32_t lm = key[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) lm = max(lm, key[j]);
    const uint32_t m = wave_max_u32(lm);
    int jw = 0, lw = 0;
#pragma unroll
    for (int j = EPL - 1; j >= 0; --j) {
      const uint64_t b = __ballot(key[j] == m);
      if (b) {
        jw = j;
        lw = __builtin_ctzll(b);
      }
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (j == jw && lane == lw) key[j] = 0u;
    if (lane == r) {
      mine = m;
      mine_id = jw * 64 + lw;
    }
  }
  const float lj = key_logit(mine);
  const float l0 = __shfl(lj, 0, 64);
  const float ex = (lane < k) ? expf(lj - l0) : 0.0f;
  const float den = wave_sum_f32(ex);
  id = (lane < k) ? mine_id : -1;
  wt = (lane < k) ? ex / den : 0.0f;
}

constexpr int kDispBlock = 1024;
constexpr int kDispWaves = kDispBlock / 64;
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

// Exclusive scan over a 1024-thread block of two values; also the totals.
__device__ __forceinline__ void block_exclusive_scan2(int v0, int v1, int& ex0, int& ex1, int& tot0, int& tot1,
                                                      int* sh /* [2 * kDispWaves] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int s0 = v0, s1 = v1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a0 = __shfl_up(s0, off, 64), a1 = __shfl_up(s1, off, 64);
    if (lane >= off) {
      s0 += a0;
      s1 += a1;
    }
  }
  if (lane == 63) {
    sh[wave] = s0;
    sh[kDispWaves + wave] = s1;
  }
  __syncthreads();
  int b0 = 0, b1 = 0, t0 = 0, t1 = 0;
  for (int w = 0; w < kDispWaves; ++w) {
    const int c0 = sh[w], c1 = sh[kDispWaves + w];
    if (w < wave) {
      b0 += c0;
      b1 += c1;
    }
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

struct DispatchLds {
  int cnt[kMaxE];
  int cursor[kMaxE];
  int scan[2 * kDispWaves];
};

// Whole stable dispatch of n assignments by one 1024-thread block.  ids may
// live in global or LDS memory.
__device__ __forceinline__ void dispatch_block(const int32_t* ids, int n, int E, int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ sorted_assign, int32_t* __restrict__ assign_pos,
                                               int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                                               DispatchLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < E) L.cnt[tid] = 0;
  __syncthreads();
  for (int a = tid; a < n; a += kDispBlock) {
    const int e = ids[a];
    if ((unsigned)e < (unsigned)E) atomicAdd(&L.cnt[e], 1);
  }
  __syncthreads();
  offsets_and_active(L.cnt, E, offsets, L.cursor, active, n_active, L.scan);
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int base = 0; base < n; base += kDispBlock) {
    const int a = base + tid;
    const bool valid = a < n;
    const int e = valid ? ids[a] : -1;
    const bool ok = valid && (unsigned)e < (unsigned)E;
    const uint64_t peers = match_peers(ok ? e : kSentinel);
    const int rank = __popcll(peers & lt), cnt_w = __popcll(peers);
    const int nw = (int)min((int64_t)kDispWaves, ceil_div(n - base, 64));
    for (int w = 0; w < nw; ++w) {
      if (wave == w && ok) {
        const int pos = L.cursor[e] + rank;
        sorted_assign[pos] = a;
        assign_pos[a] = pos;
        if (rank == cnt_w - 1) L.cursor[e] = pos + 1;
      }
      __syncthreads();
    }
    if (valid && !ok) assign_pos[a] = -1;
  }
}

}  // namespace dev
}  // namespace moe
