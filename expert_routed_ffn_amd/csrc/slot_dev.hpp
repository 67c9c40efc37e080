// slot_dev.hpp -- the resident-expert slot policy as a workgroup routine, shared
// by the stand-alone device resolve and the decode router that resolves right
// after routing.
//
// Strata feature (tech.hub77a.com), section "2. 왜 대단한가" (2): routed experts
// that are resident are used at once, the others are first moved in from host
// RAM; the most-called ones stay resident.  Policy: least recently used over
// (layer, expert), kept as a use stamp per slot (a counter that every touch
// advances; the least recently used slot has the smallest stamp).  A resolve
// stamps the hits in active order, then gives each miss, in ascending expert
// id, the slot with the smallest stamp: every slot of this resolve has a
// larger stamp than all others, so none is a victim while n_active <= n_slots.
// The (slot, blob) pairs of the misses are listed for the copy (a copy kernel,
// or the gate/up launch that stages them).
#pragma once

#include <cstdint>

#include "internal.hpp"

namespace moe {

struct SlotDevArgs {
  int32_t* map;      // [L*E] slot of (l, e) or -1
  int32_t* owner;    // [n_slots] l*E + e or -1
  int64_t* stamp;    // [n_slots] last use
  int64_t* clock;    // [1] stamps handed out so far
  uint64_t* stats;   // [5] hits, misses, bytes_h2d, resolves, evictions
  int32_t* copies;   // [2 * E] (slot, l*E + e) of the last resolve's misses
  int32_t* ncopies;  // [1]
  int E, n_slots;
  uint64_t expert_bytes;
};

namespace dev {

template <int NT_BLOCK>
struct SlotLds {
  int miss[kMaxE];
  int hits[NT_BLOCK / 64], misses[NT_BLOCK / 64];
  int64_t v[NT_BLOCK / 64];
  int i[NT_BLOCK / 64];
};

// Resolve active[0 .. n) (ascending expert ids, n <= NT_BLOCK and <= n_slots)
// of `layer`.  active may live in LDS or global memory.  All NT_BLOCK threads
// call it; it contains barriers.
template <int NT_BLOCK>
__device__ __forceinline__ void slot_resolve_block(const SlotDevArgs& a, int layer, const int32_t* active, int n,
                                                   SlotLds<NT_BLOCK>& S) {
  constexpr int NW = NT_BLOCK / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t clock = *a.clock;
  const int64_t base = (int64_t)layer * a.E;
  const bool valid = tid < n;
  const int e = valid ? active[tid] : 0;
  const int s = valid ? a.map[base + e] : -1;
  const bool hit = valid && s >= 0, miss = valid && s < 0;
  const uint64_t bh = __ballot(hit), bm = __ballot(miss);
  const uint64_t below = (1ull << lane) - 1ull;
  if (lane == 0) {
    S.hits[wave] = __popcll(bh);
    S.misses[wave] = __popcll(bm);
  }
  __syncthreads();
  int hb = 0, mb = 0, nh = 0, nm = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) {
      hb += S.hits[w];
      mb += S.misses[w];
    }
    nh += S.hits[w];
    nm += S.misses[w];
  }
  if (hit) a.stamp[s] = clock + 1 + hb + __popcll(bh & below);
  if (miss) S.miss[mb + __popcll(bm & below)] = e;
  __syncthreads();
  uint64_t evictions = 0;
  for (int j = 0; j < nm; ++j) {  // victim: the smallest stamp
    int64_t bv = INT64_MAX;
    int bi = 0;
    for (int q = tid; q < a.n_slots; q += NT_BLOCK) {
      const int64_t v = a.stamp[q];
      if (v < bv) {
        bv = v;
        bi = q;
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const int64_t ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov < bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      S.v[wave] = bv;
      S.i[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < NW; ++w)
        if (S.v[w] < bv || (S.v[w] == bv && S.i[w] < bi)) {
          bv = S.v[w];
          bi = S.i[w];
        }
      const int old = a.owner[bi];
      if (old >= 0) {
        a.map[old] = -1;
        ++evictions;
      }
      const int idx = (int)(base + S.miss[j]);
      a.owner[bi] = idx;
      a.map[idx] = bi;
      a.stamp[bi] = clock + 1 + nh + j;
      a.copies[2 * j] = bi;
      a.copies[2 * j + 1] = idx;
    }
    __syncthreads();
  }
  if (tid == 0) {
    *a.clock = clock + nh + nm;
    *a.ncopies = nm;
    a.stats[0] += (uint64_t)nh;
    a.stats[1] += (uint64_t)nm;
    a.stats[2] += (uint64_t)nm * a.expert_bytes;
    a.stats[3] += 1;
    a.stats[4] += evictions;
  }
}

}  // namespace dev
}  // namespace moe
