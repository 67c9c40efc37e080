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


__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each 16-lane row, in every lane of the row: quad swaps, then the
// half-row and row mirrors (each pairs a lane with one in the other half).
__device__ __forceinline__ float row_sum_f32(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x141>(v);
  v += dppf<0x140>(v);
  return v;
}

// Wave-private LDS of route_token: the candidates, then the k selected in order.
struct TopkLds {
  __align__(16) uint32_t key[64];
  __align__(16) int32_t id[64];
  uint32_t skey[kMaxK];
  int32_t sid[kMaxK];
};

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// One token's routing by one wave.  Lane j < k returns the j-th selected id
// in *id and its weight in *wt; other lanes return id = -1.  Expert e sits in
// lane e % 64, slot e / 64; keys are compared as (key descending, id ascending).
//
// Threshold first: tau = the k-th largest of the 64 lane maxima (a bitwise
// search, two bits per step, on ballot counts).  The k lanes whose maximum is
// at least tau hold k keys >= tau, so every key of the top k is >= tau.  The
// candidates (keys >= tau, usually little more than k) are compacted into LDS,
// each ranks itself against all of them, and the first k land in order.  If
// ties make the candidates more than 64, k rounds of "wave maximum, lowest id
// holding it, clear it" select instead.  Both give the exact top k.
template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int& id, float& wt,
                                            TopkLds& S) {
  const int lane = threadIdx.x & 63;
  // all loads first (clamped index, no branch around them), then the keys
  float lv[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) lv[j] = row[min(lane + 64 * j, E - 1)];
  uint32_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) key[j] = (lane + 64 * j < E) ? order_key(lv[j]) : 0u;
  uint32_t lm = key[0];
#pragma unroll
  for (int j = 1; j < EPL; ++j) lm = max(lm, key[j]);
  // Only the top 16 bits are searched: tau (low bits zero) is then at most
  // the k-th lane maximum, which keeps the superset property; keys within
  // one step of the 16-bit grid below it only add candidates.
  uint32_t tau = 0;  // >= 1 << 16 at the end: at least k lanes hold a finite key
#pragma unroll
  for (int b = 30; b >= 16; b -= 2) {
    const uint32_t c1 = tau | (1u << b), c2 = tau | (2u << b), c3 = tau | (3u << b);
    const int n1 = __popcll(__ballot(lm >= c1)), n2 = __popcll(__ballot(lm >= c2)), n3 = __popcll(__ballot(lm >= c3));
    tau = n3 >= k ? c3 : n2 >= k ? c2 : n1 >= k ? c1 : tau;
  }
  uint64_t cm[EPL];
  int base[EPL], cnt = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    cm[j] = __ballot(key[j] >= tau);
    base[j] = cnt;
    cnt += __popcll(cm[j]);
  }
  uint32_t mine = 0;
  int mine_id = -1;
  if (cnt <= 64) {
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if ((cm[j] >> lane) & 1ull) {
        const int pos = base[j] + lanes_below(cm[j]);
        S.key[pos] = key[j];
        S.id[pos] = lane + 64 * j;
      }
    __builtin_amdgcn_wave_barrier();
    if (lane < cnt) {
      const uint32_t mk = S.key[lane];
      const int mi = S.id[lane];
      int rank = 0;
      for (int c = 0; c < cnt; c += 4) {  // c + 3 <= 63
        const uint4 ck = *reinterpret_cast<const uint4*>(&S.key[c]);
        const int4 ci = *reinterpret_cast<const int4*>(&S.id[c]);
        const uint32_t kk[4] = {ck.x, ck.y, ck.z, ck.w};
        const int ii[4] = {ci.x, ci.y, ci.z, ci.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          rank += (c + q < cnt) & ((kk[q] > mk) | ((kk[q] == mk) & (ii[q] < mi)));
      }
      if (rank < k) {
        S.skey[rank] = mk;
        S.sid[rank] = mi;
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < k) {
      mine = S.skey[lane];
      mine_id = S.sid[lane];
    }
    __builtin_amdgcn_wave_barrier();
  } else {
    for (int r = 0; r < k; ++r) {
      uint32_t bm = key[0];
#pragma unroll
      for (int j = 1; j < EPL; ++j) bm = max(bm, key[j]);
      int jl = EPL - 1;
#pragma unroll
      for (int j = EPL - 2; j >= 0; --j) jl = key[j] == bm ? j : jl;
      const uint32_t m = wave_max_u32(bm);
      const uint32_t w = wave_min_u32(bm == m ? (uint32_t)(jl * 64 + lane) : 0xFFFFFFFFu);
      const int clr = lane == (int)(w & 63) ? jl : -1;
#pragma unroll
      for (int j = 0; j < EPL; ++j) key[j] = clr == j ? 0u : key[j];
      if (lane == r) {
        mine = m;
        mine_id = (int)w;
      }
    }
  }
  const float lj = key_logit(mine);
  const float l0 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, lj)));
  const float ex = (lane < k) ? expf(lj - l0) : 0.0f;
  const float den = row_sum_f32(ex);  // k <= 16: every term sits in lanes 0..15
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


// ---- decode router: routing, grouping and descriptors in one workgroup -------------
// For n = T*k <= kDecodeMaxN assignments.  Route all T tokens (one wave per
// token), then the stable grouping of moe_dispatch done in LDS: the position
// of assignment a is the number of assignments before it in (expert, index)
// order; an assignment that is the first of its expert opens an active slot,
// numbered by the count of such first assignments with a lower expert id.
// decode_route_lds leaves all of it in LDS; decode_route_write then writes
// every output of moe_route_topk and moe_dispatch, one descriptor per slot
// (expert, first position, row count, tokens, assignments; e = -1 for slots
// past n_active) and the (expert, assignment) pair of every sorted position.
// The fused decode gate/up kernel runs the first part in every workgroup and
// the second in one.
constexpr int kDecodeMaxN = kDescT * kMaxK;  // 192
constexpr int kNoId = 0x7FFFFFFF;

struct RouterLds {
  __align__(16) int32_t id[kDecodeMaxN];
  __align__(16) int32_t first_e[kDecodeMaxN];  // expert id if the first of its expert, else kNoId
  float w[kDecodeMaxN];
  int32_t sorted[kDecodeMaxN];
  int32_t pos[kDecodeMaxN];
  int32_t slot_e[kDecodeMaxN], slot_p0[kDecodeMaxN], slot_ne[kDecodeMaxN];
  uint32_t bits[kMaxE / 32];  // experts present (route_ids_lds)
  int32_t na;
  TopkLds tk[kDescT];  // one per routing wave (wave index < T <= kDescT)
};

// Counts over the n ids in LDS (padded with kNoId to a multiple of 8), eight
// ids per step in two 128-bit reads so the reads overlap:
//   less += ids < e, before += (ids == e and index < a), same += ids == e.
__device__ __forceinline__ void count_ids(const int32_t* s_id, int n8, int e, int a, int& less, int& before,
                                          int& same) {
  less = before = same = 0;
  for (int b = 0; b < n8; b += 8) {
    const int4 u = *reinterpret_cast<const int4*>(s_id + b);
    const int4 v = *reinterpret_cast<const int4*>(s_id + b + 4);
    const int q[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      less += q[i] < e;
      same += q[i] == e;
      before += (q[i] == e) & (b + i < a);
    }
  }
}

// Routing and grouping into L.  Ends with a barrier: L is complete for every thread.
template <int EPL, int NT_BLOCK>
__device__ __forceinline__ void decode_route_lds(const float* __restrict__ logits, int T, int E, int k,
                                                 RouterLds& L) {
  constexpr int NW = NT_BLOCK / 64;
  constexpr int R = (kDecodeMaxN + NT_BLOCK - 1) / NT_BLOCK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = T * k, n8 = (n + 7) & ~7;
  for (int t = wave; t < T; t += NW) {
    int id;
    float wt;
    route_token<EPL>(logits + (size_t)t * E, E, k, id, wt, L.tk[wave]);
    if (lane < k) {
      L.id[t * k + lane] = id;
      L.w[t * k + lane] = wt;
    }
  }
  for (int i = n + tid; i < n8; i += NT_BLOCK) L.id[i] = kNoId;
  __syncthreads();
  for (int a = tid; a < n8; a += NT_BLOCK) {
    if (a < n) {
      const int e = L.id[a];
      int less, before, same;
      count_ids(L.id, n8, e, a, less, before, same);
      const int pos = less + before;
      L.sorted[pos] = a;
      L.pos[a] = pos;
      L.first_e[a] = before == 0 ? e : kNoId;
      if (before == 0) {  // first of its expert: its position opens the expert's rows
        L.slot_p0[a] = pos;
        L.slot_ne[a] = same;
      }
    } else {
      L.first_e[a] = kNoId;
    }
  }
  __syncthreads();
  // slot of each first-of-expert assignment = number of first assignments with a lower expert id
  int slot[R], p0[R], ne[R], e0[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int a = tid + r * NT_BLOCK;
    slot[r] = -1;
    if (a < n && L.first_e[a] != kNoId) {
      e0[r] = L.first_e[a];
      int less, before, same;
      count_ids(L.first_e, n8, e0[r], 0, less, before, same);
      slot[r] = less;
      p0[r] = L.slot_p0[a];
      ne[r] = L.slot_ne[a];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (slot[r] >= 0) {
      L.slot_e[slot[r]] = e0[r];
      L.slot_p0[slot[r]] = p0[r];
      L.slot_ne[slot[r]] = ne[r];
    }
  if (wave == 0) {
    int c = 0;
    for (int b = lane; b < n; b += 64) c += L.first_e[b] != kNoId;
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
    if (lane == 0) L.na = c;
  }
  __syncthreads();
}

// Routing only, for workgroups that then read their slot with wave_slot:
// L.id (padded with kNoId to kDecodeMaxN) and the bitmap of the experts
// present.  Ends with a barrier.
template <int EPL, int NT_BLOCK>
__device__ __forceinline__ void route_ids_lds(const float* __restrict__ logits, int T, int E, int k, RouterLds& L) {
  constexpr int NW = NT_BLOCK / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = T * k;
  if (tid < kMaxE / 32) L.bits[tid] = 0u;
  for (int i = n + tid; i < kDecodeMaxN; i += NT_BLOCK) L.id[i] = kNoId;
  __syncthreads();
  for (int t = wave; t < T; t += NW) {
    int id;
    float wt;
    route_token<EPL>(logits + (size_t)t * E, E, k, id, wt, L.tk[wave]);
    if (lane < k) {
      L.id[t * k + lane] = id;
      atomicOr(&L.bits[id >> 5], 1u << (id & 31));
    }
  }
  __syncthreads();
}

template <int CTRL>
__device__ __forceinline__ int dpp_shr(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

// One active slot as a wave sees it: expert (-1 past the active experts),
// first sorted position, row count, and in lane j < min(ne, 64) the token of
// the slot's j-th row.
struct WaveSlot {
  int e, p0, ne, tokv;
};

// Slot s from route_ids_lds's result, computed by each wave on its own (no
// barrier): the active experts are the set bits of the bitmap in ascending
// id, so slot s is its s-th set bit (prefix counts over the bitmap words);
// its first position is the number of assignments to lower ids and its rows
// are its assignments in ascending index, the order of the stable dispatch.
__device__ __forceinline__ WaveSlot wave_slot(const RouterLds& L, int s, int k) {
  static_assert(kMaxE / 32 == 32 && kDecodeMaxN <= 192, "bitmap words fit one half-wave; ids three per lane");
  const int lane = threadIdx.x & 63;
  const uint32_t bw = lane < 32 ? L.bits[lane] : 0u;
  const int c = __popc(bw);
  int incl = c;  // inclusive prefix over the 32 words: within 16-lane rows, then across
  incl += dpp_shr<0x111>(incl);
  incl += dpp_shr<0x112>(incl);
  incl += dpp_shr<0x114>(incl);
  incl += dpp_shr<0x118>(incl);
  const int row0 = __builtin_amdgcn_readlane(incl, 15);
  if (lane >= 16) incl += row0;
  const int na = __builtin_amdgcn_readlane(incl, 31);
  WaveSlot r{-1, 0, 0, 0};
  if (s >= na) return r;
  const int ls = __popcll(__ballot(lane < 32 && incl <= s));  // word holding the s-th bit
  const int rr = s - (__builtin_amdgcn_readlane(incl, ls) - __builtin_amdgcn_readlane(c, ls));
  const uint32_t word = (uint32_t)__builtin_amdgcn_readlane((int)bw, ls);
  const uint32_t below = lane < 32 ? word & ((1u << (lane & 31)) - 1u) : 0u;
  const bool hit = lane < 32 && ((word >> (lane & 31)) & 1u) && __popc(below) == rr;
  const int e = 32 * ls + __builtin_ctzll(__ballot(hit));
  const int i0 = L.id[lane], i1 = L.id[lane + 64], i2 = L.id[lane + 128];
  uint64_t m0 = __ballot(i0 == e), m1 = __ballot(i1 == e), m2 = __ballot(i2 == e);
  r.e = e;
  r.p0 = __popcll(__ballot(i0 < e)) + __popcll(__ballot(i1 < e)) + __popcll(__ballot(i2 < e));
  r.ne = __popcll(m0) + __popcll(m1) + __popcll(m2);
  int asg = 0;
  const int nl = min(r.ne, 64);
  for (int j = 0; j < nl; ++j) {
    int a;
    if (m0) {
      a = __builtin_ctzll(m0);
      m0 &= m0 - 1;
    } else if (m1) {
      a = 64 + __builtin_ctzll(m1);
      m1 &= m1 - 1;
    } else {
      a = 128 + __builtin_ctzll(m2);
      m2 &= m2 - 1;
    }
    if (lane == j) asg = a;
  }
  r.tokv = asg / k;
  return r;
}

// Slot s of L as a descriptor (e = -1 past n_active).
__device__ __forceinline__ SlotDesc slot_desc(const RouterLds& L, int s, int k) {
  const int na = L.na;
  SlotDesc d;
  d.e = s < na ? L.slot_e[s] : -1;
  d.p0 = s < na ? L.slot_p0[s] : 0;
  d.ne = s < na ? L.slot_ne[s] : 0;
  d.pad = 0;
  for (int j = 0; j < kDescT; ++j) {
    const int a = j < d.ne ? L.sorted[d.p0 + j] : 0;
    d.asg[j] = a;
    d.tok[j] = a / k;
  }
  for (int j = 0; j < 4; ++j) d.pad2[j] = 0;
  return d;
}

// Global outputs from a complete L (no barrier inside).
template <int NT_BLOCK>
__device__ __forceinline__ void decode_route_write(const RouterLds& L, int T, int E, int k,
                                                   int32_t* __restrict__ ids, float* __restrict__ w,
                                                   int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_assign,
                                                   int32_t* __restrict__ assign_pos, int32_t* __restrict__ active,
                                                   int32_t* __restrict__ n_active, SlotDesc* __restrict__ desc,
                                                   int max_active, int32_t* __restrict__ rows,
                                                   int32_t* __restrict__ nrows) {
  const int tid = threadIdx.x;
  const int n = T * k, n8 = (n + 7) & ~7, na = L.na;
  for (int a = tid; a < n; a += NT_BLOCK) {
    ids[a] = L.id[a];
    w[a] = L.w[a];
    assign_pos[a] = L.pos[a];
  }
  for (int p = tid; p < n; p += NT_BLOCK) {
    const int a = L.sorted[p];
    sorted_assign[p] = a;
    rows[2 * p] = L.id[a];
    rows[2 * p + 1] = a;
  }
  for (int s2 = tid; s2 < na; s2 += NT_BLOCK) active[s2] = L.slot_e[s2];
  if (tid == 0) {
    *n_active = na;
    *nrows = n;
  }
  if (desc)
    for (int s2 = tid; s2 < max_active; s2 += NT_BLOCK) desc[s2] = slot_desc(L, s2, k);
  for (int e = tid; e <= E; e += NT_BLOCK) {
    int less, before, same;
    count_ids(L.id, n8, e, 0, less, before, same);
    offsets[e] = less;
  }
}

}  // namespace dev
}  // namespace moe
