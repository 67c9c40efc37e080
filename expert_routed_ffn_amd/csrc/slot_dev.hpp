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
#include "route_dispatch_dev.hpp"

namespace moe {

struct SlotDevArgs {
  int32_t* map;      // [L*E] slot of (l, e) or -1
  int32_t* owner;    // [n_slots] l*E + e or -1
  int64_t* stamp;    // [n_slots] last use
  int64_t* clock;    // [1] stamps handed out so far
  uint64_t* stats;   // [5] hits, misses, bytes_h2d, resolves, evictions
  int32_t* copies;   // [2 * E] (slot, l*E + e) of the last resolve's misses
  int32_t* ncopies;  // [1]
  uint64_t* ready;   // [1] clock + 1 once a resolve inside a gate/up launch has published its record
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

// ---- the same resolve inside a launch that uses its outcome ------------------------
// In a gate/up launch that resolves the step's experts itself, workgroup 0
// resolves (slot_resolve_publish) while the other workgroups run.  It writes
// the stamps and owners at once (only a resolve reads them) but leaves the
// map, the clock, the miss list and the counters as they were, since the
// other workgroups of the launch look routed experts up in the map and read
// the clock; it records what those need (kSlotRecordWords int32 words, in the
// caller's workspace) and then sets the table's ready word to clock + 1.  A
// workgroup whose expert is in the map uses that slot at once; one whose
// expert is not waits for the ready word and takes its slot from the record.
// A workgroup of the next launch writes the rest (slot_record_commit).  The
// outcome equals slot_resolve_block's.
//
// Record layout: n, nh, nm, clock (low, high word), then kDecodeMaxN words
// each of: slot of active expert s, victim slot of miss j, blob l*E + e of
// miss j, previous owner of that victim slot.
constexpr int kSlotRecordWords = 5 + 4 * kDecodeMaxN;
constexpr int kRecSlot = 5, kRecMissSlot = 5 + kDecodeMaxN, kRecMissIdx = 5 + 2 * kDecodeMaxN,
              kRecOldOwner = 5 + 3 * kDecodeMaxN;
constexpr int kResolveRegs = 16;  // stamps held per thread (tables up to NT_BLOCK * 16 slots)

template <int NT_BLOCK>
struct ResolveLds {
  int mapl[kMaxE];  // the layer's map row
  int slot[kDecodeMaxN], rank[kDecodeMaxN];
  uint32_t hitbits[NT_BLOCK * kResolveRegs / 32];
  int nh, nm;
  int64_t rv[NT_BLOCK / 64];
  int ri[NT_BLOCK / 64];
};

// Loads issued before the routing so that their latency overlaps it: the
// layer's map row and, for tables of up to NT_BLOCK * kResolveRegs slots, the
// stamps (thread t holds slots t, t + NT_BLOCK, ...).
template <int NT_BLOCK>
struct ResolvePrefetch {
  int mv[kMaxE / NT_BLOCK];
  int64_t r[kResolveRegs];
};

template <int NT_BLOCK>
__device__ __forceinline__ void slot_prefetch_map(const SlotDevArgs& a, int layer, ResolvePrefetch<NT_BLOCK>& P) {
  const int64_t base = (int64_t)layer * a.E;
#pragma unroll
  for (int u = 0; u < kMaxE / NT_BLOCK; ++u) {
    const int e = threadIdx.x + u * NT_BLOCK;
    P.mv[u] = e < a.E ? a.map[base + e] : -1;
  }
}

template <int NT_BLOCK>
__device__ __forceinline__ void slot_prefetch_stamps(const SlotDevArgs& a, ResolvePrefetch<NT_BLOCK>& P) {
  if (a.n_slots > NT_BLOCK * kResolveRegs) return;
#pragma unroll
  for (int u = 0; u < kResolveRegs; ++u) {
    const int q = threadIdx.x + u * NT_BLOCK;
    P.r[u] = q < a.n_slots ? a.stamp[q] : INT64_MAX;
  }
}

// The prefetched map row into LDS (the caller synchronises before reading it).
template <int NT_BLOCK>
__device__ __forceinline__ void slot_map_to_lds(const ResolvePrefetch<NT_BLOCK>& P, int* mapl) {
#pragma unroll
  for (int u = 0; u < kMaxE / NT_BLOCK; ++u) mapl[threadIdx.x + u * NT_BLOCK] = P.mv[u];
}

// act: active experts of `layer` in ascending id (LDS), n of them (1 <= n <=
// kDecodeMaxN, n <= n_slots); P from slot_prefetch_map and
// slot_prefetch_stamps.  All threads call it; it contains barriers.
template <int NT_BLOCK>
__device__ __forceinline__ void slot_resolve_publish(const SlotDevArgs& a, int layer, const int32_t* act, int n,
                                                     int32_t* rec, ResolvePrefetch<NT_BLOCK>& P,
                                                     ResolveLds<NT_BLOCK>& S) {
  constexpr int NW = NT_BLOCK / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t base = (int64_t)layer * a.E;
  const int64_t clock = *a.clock;
  const bool in_regs = a.n_slots <= NT_BLOCK * kResolveRegs;
  slot_map_to_lds(P, S.mapl);
  for (int w = tid; w < NT_BLOCK * kResolveRegs / 32; w += NT_BLOCK) S.hitbits[w] = 0u;
  __syncthreads();
  for (int s = tid; s < n; s += NT_BLOCK) {
    const int q = S.mapl[act[s]];
    S.slot[s] = q;
    if (q >= 0 && in_regs) atomicOr(&S.hitbits[q >> 5], 1u << (q & 31));
  }
  __syncthreads();
  if (wave == 0) {  // hits take the next stamps in active order
    int nh = 0, nm = 0;
    for (int s0 = 0; s0 < n; s0 += 64) {
      const int s = s0 + lane;
      const bool valid = s < n, hit = valid && S.slot[s] >= 0, miss = valid && S.slot[s] < 0;
      const uint64_t bh = __ballot(hit), bm = __ballot(miss), below = (1ull << lane) - 1ull;
      if (hit) {
        S.rank[s] = nh + __popcll(bh & below);
        if (!in_regs) a.stamp[S.slot[s]] = clock + 1 + S.rank[s];
      }
      if (miss) S.rank[s] = nm + __popcll(bm & below);
      nh += __popcll(bh);
      nm += __popcll(bm);
    }
    if (lane == 0) {
      S.nh = nh;
      S.nm = nm;
    }
  }
  __syncthreads();  // no hit is a victim: masked in the registers, or its new stamp exceeds every other
  const int nh = S.nh, nm = S.nm;
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kResolveRegs; ++u) {
      const int q = tid + u * NT_BLOCK;
      if ((S.hitbits[q >> 5] >> (q & 31)) & 1u) P.r[u] = INT64_MAX;
    }
  }
  int js = 0;  // active index of miss j
  for (int j = 0; j < nm; ++j) {
    while (S.slot[js] >= 0) ++js;  // misses in ascending expert id
    int64_t bv = INT64_MAX;
    int bi = 0x7FFFFFFF;
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kResolveRegs; ++u)
        if (P.r[u] < bv) {
          bv = P.r[u];
          bi = tid + u * NT_BLOCK;
        }
    } else {
      for (int q0 = tid; q0 < a.n_slots; q0 += NT_BLOCK * kResolveRegs) {
        int64_t v[kResolveRegs];
#pragma unroll
        for (int u = 0; u < kResolveRegs; ++u) {
          const int q = q0 + u * NT_BLOCK;
          v[u] = q < a.n_slots ? a.stamp[q] : INT64_MAX;
        }
#pragma unroll
        for (int u = 0; u < kResolveRegs; ++u)
          if (v[u] < bv) {
            bv = v[u];
            bi = q0 + u * NT_BLOCK;
          }
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
      S.rv[wave] = bv;
      S.ri[wave] = bi;
    }
    __syncthreads();
    bv = S.rv[0];
    bi = S.ri[0];
    for (int w = 1; w < NW; ++w)
      if (S.rv[w] < bv || (S.rv[w] == bv && S.ri[w] < bi)) {
        bv = S.rv[w];
        bi = S.ri[w];
      }
    if (tid == 0) {
      S.slot[js] = bi;
      if (!in_regs) a.stamp[bi] = clock + 1 + nh + j;
    }
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kResolveRegs; ++u)
        if (tid + u * NT_BLOCK == bi) P.r[u] = INT64_MAX;
    }
    __syncthreads();
    ++js;
  }
  // the record, then the ready word; the rest of this resolve's writes after it
  if (tid == 0) {
    rec[0] = n;
    rec[1] = nh;
    rec[2] = nm;
    rec[3] = (int32_t)(uint32_t)((uint64_t)clock & 0xFFFFFFFFu);
    rec[4] = (int32_t)(uint32_t)((uint64_t)clock >> 32);
  }
  for (int s = tid; s < n; s += NT_BLOCK) {
    rec[kRecSlot + s] = S.slot[s];
    if (S.mapl[act[s]] < 0) {  // the miss list: victim slot and blob of the j-th miss (ascending expert id)
      const int j = S.rank[s];
      rec[kRecMissSlot + j] = S.slot[s];
      rec[kRecMissIdx + j] = (int)(base + act[s]);
    }
  }
  __threadfence();  // this thread's record words before the ready word
  __syncthreads();
  if (tid == 0) __hip_atomic_store(a.ready, (uint64_t)clock + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  for (int s = tid; s < n; s += NT_BLOCK) {
    const int q = S.slot[s];
    if (S.mapl[act[s]] >= 0) {  // a hit: its new stamp
      if (in_regs) a.stamp[q] = clock + 1 + S.rank[s];
    } else {  // a victim: new owner and stamp, the old owner for the map update
      const int j = S.rank[s];
      rec[kRecOldOwner + j] = a.owner[q];
      a.owner[q] = (int)(base + act[s]);
      if (in_regs) a.stamp[q] = clock + 1 + nh + j;
    }
  }
}

// Waits (thread 0; the others at the barrier) until the resolve of this launch
// has published, at most about 0.1 s; false if it has not by then (the
// caller's outputs are then marked invalid rather than waiting on).
__device__ __forceinline__ bool slot_wait_published(const SlotDevArgs& a, int64_t clock, int* lds_flag) {
  if (threadIdx.x == 0) {
    const uint64_t want = (uint64_t)clock + 1;
    int ok = 0;
    for (int it = 0; it < (1 << 20); ++it) {
      if (__hip_atomic_load(a.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want) {
        ok = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // order the record reads after the ready word
    *lds_flag = ok;
  }
  __syncthreads();
  return *lds_flag != 0;
}

// A published record word, read past any stale cache line.
__device__ __forceinline__ int rec_word(const int32_t* rec, int i) {
  return __hip_atomic_load(rec + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Writes the rest of the recorded resolve into the table state: the map
// (evicted owners out, misses in), the clock, the miss list and the counters.
// One thread, in a launch after the one that resolved.
__device__ __forceinline__ void slot_record_commit(const SlotDevArgs& a, const int32_t* rec) {
  const int nh = rec[1], nm = rec[2];
  const int64_t clock = (int64_t)(((uint64_t)(uint32_t)rec[4] << 32) | (uint32_t)rec[3]);
  uint64_t evictions = 0;
  for (int j = 0; j < nm; ++j) {
    const int v = rec[kRecMissSlot + j], idx = rec[kRecMissIdx + j], old = rec[kRecOldOwner + j];
    if (old >= 0) {
      a.map[old] = -1;
      ++evictions;
    }
    a.map[idx] = v;
    a.copies[2 * j] = v;
    a.copies[2 * j + 1] = idx;
  }
  *a.clock = clock + nh + nm;
  *a.ncopies = nm;
  a.stats[0] += (uint64_t)nh;
  a.stats[1] += (uint64_t)nm;
  a.stats[2] += (uint64_t)nm * a.expert_bytes;
  a.stats[3] += 1;
  a.stats[4] += evictions;
}

}  // namespace dev
}  // namespace moe
