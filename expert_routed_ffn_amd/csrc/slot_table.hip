// slot_table.hip -- resident-expert slot table (host side).
//
// Strata feature (tech.hub77a.com), section "2. 왜 대단한가" (2): the most-called
// experts stay resident in GPU memory and all of them sit in host RAM; a
// routed expert that is resident is used at once, any other is first moved in
// from RAM.  Janas-LLM item (onedev.kr/items/2196): experts that come back are
// kept cached.  Strata feature, section "3. 바로 써먹기": part of host memory is
// locked for the graphics card at load time.
//
// The table owns the placement of L*E (layer, expert) blobs in n_slots device
// slots.  The policy is least-recently-used over (layer, expert), kept as an
// index-linked list of slots (head = least recently used).  A resolve first
// marks every hit as most recently used, then serves the misses in ascending
// expert id, each taking the list head as victim; since every slot used by the
// current resolve has just moved to the tail, a victim is never one of them
// (n_active <= n_slots is checked first).
//
// Copies go straight from the page-locked master copy into the victim slot
// with hipMemcpyAsync on the caller's stream, so the FFN kernels enqueued after
// the resolve see them.
//
// Device mode (moe_slot_table_enable_device): the same policy runs on the GPU
// so that a resolve needs no host round trip.  LRU order is kept as a use
// stamp per slot (a counter that every touch advances, so the least recently
// used slot is the one with the smallest stamp; stamps are unique).  One
// workgroup stamps the hits in active order, then gives each miss, in
// ascending expert id, the slot of smallest stamp; a second kernel copies the
// missed blobs from the page-locked master copy (read through its device
// mapping) into their slots.  Both kernels are ordered on the caller's stream
// and can be captured in a graph.  The device map is re-uploaded from a page-locked
// mirror; a resolve waits for the stream before touching the mirror, so the
// previous upload has always completed before the mirror is modified (no
// staging buffer is reused while a copy from it may be in flight).
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "internal.hpp"
#include "slot_dev.hpp"

struct moe_slot_table {
  int L = 0, E = 0, n_slots = 0;
  size_t expert_bytes = 0;
  bool host_only = false;
  // device mode
  const uint8_t* host = nullptr;  // page-locked master copy [L*E*expert_bytes]
  uint8_t* slots = nullptr;       // device [n_slots*expert_bytes]
  int32_t* slot_map_dev = nullptr;
  int32_t* map_mirror = nullptr;  // page-locked [L*E]
  int32_t* act_stage = nullptr;   // page-locked [E + 1]
  // host-only mode
  moe_copy_fn copy_fn = nullptr;
  void* user = nullptr;
  // policy state
  std::vector<int32_t> map;    // [L*E] slot or -1
  std::vector<int32_t> owner;  // [n_slots] l*E + e or -1
  std::vector<int32_t> prev, next;
  int32_t head = -1, tail = -1;
  moe_slot_stats stats{};
  // device mode (state in caller memory)
  bool device_mode = false;
  const uint8_t* host_dev = nullptr;  // device mapping of `host`
  int32_t* d_owner = nullptr;         // [n_slots] l*E + e or -1
  int64_t* d_stamp = nullptr;         // [n_slots] last use
  int64_t* d_clock = nullptr;         // [1] stamps handed out so far
  uint64_t* d_stats = nullptr;        // [5] hits, misses, bytes_h2d, resolves, evictions
  int32_t* d_copies = nullptr;        // [2 * E] (slot, l*E + e) of the last resolve's misses
  int32_t* d_ncopies = nullptr;       // [1]
  uint64_t* d_ready = nullptr;        // [1] see SlotDevArgs::ready
};

namespace {

using moe::fail;

void lru_unlink(moe_slot_table* t, int s) {
  const int p = t->prev[s], n = t->next[s];
  if (p >= 0) t->next[p] = n; else t->head = n;
  if (n >= 0) t->prev[n] = p; else t->tail = p;
  t->prev[s] = t->next[s] = -1;
}

void lru_push_tail(moe_slot_table* t, int s) {
  t->prev[s] = t->tail;
  t->next[s] = -1;
  if (t->tail >= 0) t->next[t->tail] = s; else t->head = s;
  t->tail = s;
}

void lru_touch(moe_slot_table* t, int s) {
  if (t->tail == s) return;
  lru_unlink(t, s);
  lru_push_tail(t, s);
}

void init_policy(moe_slot_table* t) {
  t->map.assign((size_t)t->L * t->E, -1);
  t->owner.assign(t->n_slots, -1);
  t->prev.assign(t->n_slots, -1);
  t->next.assign(t->n_slots, -1);
  t->head = t->tail = -1;
  for (int s = 0; s < t->n_slots; ++s) lru_push_tail(t, s);  // free slots are used in ascending order
}

// Place (layer, expert) into the LRU victim slot; returns the slot.
int place(moe_slot_table* t, int layer, int expert) {
  const int s = t->head;
  const int64_t idx = (int64_t)layer * t->E + expert;
  if (t->owner[s] >= 0) {
    t->map[t->owner[s]] = -1;
    t->stats.evictions++;
  }
  t->owner[s] = (int32_t)idx;
  t->map[idx] = s;
  lru_touch(t, s);
  return s;
}

moe_status do_copy(moe_slot_table* t, int slot, int layer, int expert, hipStream_t stream) {
  t->stats.bytes_h2d += t->expert_bytes;
  if (t->host_only) {
    t->copy_fn(t->user, slot, layer, expert);
    return MOE_OK;
  }
  const uint8_t* src = t->host + ((size_t)layer * t->E + expert) * t->expert_bytes;
  uint8_t* dst = t->slots + (size_t)slot * t->expert_bytes;
  return moe::check_hip(hipMemcpyAsync(dst, src, t->expert_bytes, hipMemcpyHostToDevice, stream),
                        "slot table: expert copy");
}

moe_status upload_map(moe_slot_table* t, hipStream_t stream) {
  if (t->host_only) return MOE_OK;
  std::memcpy(t->map_mirror, t->map.data(), t->map.size() * sizeof(int32_t));
  return moe::check_hip(hipMemcpyAsync(t->slot_map_dev, t->map_mirror, t->map.size() * sizeof(int32_t),
                                       hipMemcpyHostToDevice, stream),
                        "slot table: map upload");
}

// The policy step shared by the device and host-only tables.
moe_status resolve_list(moe_slot_table* t, int layer, const int32_t* act, int n, hipStream_t stream, bool& changed) {
  changed = false;
  if (n > t->n_slots)
    return fail(MOE_ECAPACITY, "moe_slot_table_resolve: " + std::to_string(n) + " active experts, " +
                                   std::to_string(t->n_slots) + " slots");
  for (int i = 0; i < n; ++i)
    if (act[i] < 0 || act[i] >= t->E) return fail(MOE_EINVAL, "moe_slot_table_resolve: expert id out of range");
  t->stats.resolves++;
  std::vector<int32_t> misses;
  for (int i = 0; i < n; ++i) {
    const int64_t idx = (int64_t)layer * t->E + act[i];
    const int s = t->map[idx];
    if (s >= 0) {
      t->stats.hits++;
      lru_touch(t, s);
    } else {
      misses.push_back(act[i]);
    }
  }
  std::sort(misses.begin(), misses.end());
  misses.erase(std::unique(misses.begin(), misses.end()), misses.end());
  for (int e : misses) {
    t->stats.misses++;
    const int s = place(t, layer, e);
    if (moe_status st = do_copy(t, s, layer, e, stream)) return st;
    changed = true;
  }
  return MOE_OK;
}

// ---- device mode -------------------------------------------------------------------------
struct DevLayout {
  size_t owner, stamp, clock, stats, copies, ncopies, ready, bytes;
};

DevLayout dev_layout(int E, int n_slots) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  DevLayout d;
  size_t off = 0;
  d.owner = off;
  off += up((size_t)n_slots * 4);
  d.stamp = off;
  off += up((size_t)n_slots * 8);
  d.clock = off;
  off += 256;
  d.stats = off;
  off += 256;
  d.copies = off;
  off += up((size_t)E * 8);
  d.ncopies = off;
  off += 256;
  d.ready = off;
  off += 256;
  d.bytes = off;
  return d;
}

constexpr int kResolveThreads = 1024;

// One resolve in one workgroup.  n_active <= max_active <= n_slots (checked
// on the host when the call is enqueued; a larger device count is clamped).
__global__ __launch_bounds__(kResolveThreads) void slot_resolve_kernel(moe::SlotDevArgs a, int layer,
                                                                       const int32_t* __restrict__ active,
                                                                       const int32_t* __restrict__ n_active,
                                                                       int max_active) {
  __shared__ moe::dev::SlotLds<kResolveThreads> S;
  moe::dev::slot_resolve_block<kResolveThreads>(a, layer, active, min(max(*n_active, 0), max_active), S);
}

constexpr int kCopyThreads = 256, kCopyUnroll = 4;
constexpr int64_t kCopyChunk = (int64_t)kCopyThreads * 16 * kCopyUnroll;  // bytes per workgroup step

// The last resolve's misses: blob l*E + e of the master copy (device mapping
// of page-locked host memory) into its slot.  Persistent grid over
// (miss, chunk) work items.
__global__ __launch_bounds__(kCopyThreads) void slot_copy_kernel(const int32_t* __restrict__ copies,
                                                                 const int32_t* __restrict__ ncopies,
                                                                 const uint8_t* __restrict__ host_dev,
                                                                 uint8_t* __restrict__ slots, int64_t expert_bytes) {
  const int nc = *ncopies;
  const int64_t cpb = (expert_bytes + kCopyChunk - 1) / kCopyChunk;
  const int64_t total = (int64_t)nc * cpb;
  for (int64_t w = blockIdx.x; w < total; w += gridDim.x) {
    const int c = (int)(w / cpb);
    const int64_t ch = w % cpb;
    const uint8_t* src = host_dev + (int64_t)copies[2 * c + 1] * expert_bytes;
    uint8_t* dst = slots + (int64_t)copies[2 * c] * expert_bytes;
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t off = ch * kCopyChunk + ((int64_t)u * kCopyThreads + threadIdx.x) * 16;
      if (off < expert_bytes) v[u] = *reinterpret_cast<const uint4*>(src + off);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t off = ch * kCopyChunk + ((int64_t)u * kCopyThreads + threadIdx.x) * 16;
      if (off < expert_bytes) *reinterpret_cast<uint4*>(dst + off) = v[u];
    }
  }
}

constexpr int kCopyGrid = 512;

void free_table(moe_slot_table* t) {
  if (!t) return;
  if (t->map_mirror) (void)hipHostFree(t->map_mirror);
  if (t->act_stage) (void)hipHostFree(t->act_stage);
  delete t;
}

}  // namespace

extern "C" {

moe_status moe_slot_table_create(int L, int E, int n_slots, size_t expert_bytes, const void* host_experts, void* slots,
                                 int32_t* slot_map, hipStream_t stream, moe_slot_table** out) {
  if (!out) return fail(MOE_EINVAL, "moe_slot_table_create: null out");
  *out = nullptr;
  if (L < 1 || E < 1 || E > moe::kMaxE || n_slots < 1)
    return fail(MOE_EINVAL, "moe_slot_table_create: L, E or n_slots out of range");
  if (expert_bytes == 0 || expert_bytes % 256)
    return fail(MOE_EINVAL, "moe_slot_table_create: expert_bytes must be a nonzero multiple of 256");
  if (!host_experts || !slots || !slot_map) return fail(MOE_EINVAL, "moe_slot_table_create: null pointer");
  hipPointerAttribute_t attr;
  const hipError_t pe = hipPointerGetAttributes(&attr, host_experts);
  if (pe != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(MOE_ENOTPINNED, "moe_slot_table_create: host_experts is not page-locked host memory");
  }
  moe_slot_table* t = new moe_slot_table;
  t->L = L;
  t->E = E;
  t->n_slots = n_slots;
  t->expert_bytes = expert_bytes;
  t->host = static_cast<const uint8_t*>(host_experts);
  t->slots = static_cast<uint8_t*>(slots);
  t->slot_map_dev = slot_map;
  if (hipHostMalloc((void**)&t->map_mirror, sizeof(int32_t) * (size_t)L * E, hipHostMallocDefault) != hipSuccess ||
      hipHostMalloc((void**)&t->act_stage, sizeof(int32_t) * ((size_t)E + 1), hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    free_table(t);
    return fail(MOE_EHIP, "moe_slot_table_create: page-locked staging allocation failed");
  }
  init_policy(t);
  if (moe_status st = upload_map(t, stream)) {
    free_table(t);
    return st;
  }
  *out = t;
  return MOE_OK;
}

moe_status moe_slot_table_create_host(int L, int E, int n_slots, moe_copy_fn copy_fn, void* user,
                                      moe_slot_table** out) {
  if (!out) return fail(MOE_EINVAL, "moe_slot_table_create_host: null out");
  *out = nullptr;
  if (L < 1 || E < 1 || E > moe::kMaxE || n_slots < 1)
    return fail(MOE_EINVAL, "moe_slot_table_create_host: L, E or n_slots out of range");
  if (!copy_fn) return fail(MOE_EINVAL, "moe_slot_table_create_host: null copy_fn");
  moe_slot_table* t = new moe_slot_table;
  t->L = L;
  t->E = E;
  t->n_slots = n_slots;
  t->expert_bytes = 256;
  t->host_only = true;
  t->copy_fn = copy_fn;
  t->user = user;
  init_policy(t);
  *out = t;
  return MOE_OK;
}

moe_status moe_slot_table_preload(moe_slot_table* t, const int32_t* layer_expert, int n, hipStream_t stream) {
  if (!t) return fail(MOE_EINVAL, "moe_slot_table_preload: null table");
  if (t->device_mode) return fail(MOE_EINVAL, "moe_slot_table_preload: the table is in device mode");
  if (n < 0 || (n > 0 && !layer_expert)) return fail(MOE_EINVAL, "moe_slot_table_preload: bad list");
  for (int i = 0; i < n; ++i) {
    const int l = layer_expert[2 * i], e = layer_expert[2 * i + 1];
    if (l < 0 || l >= t->L || e < 0 || e >= t->E) return fail(MOE_EINVAL, "moe_slot_table_preload: pair out of range");
  }
  if (!t->host_only) {
    // the mirror and slots may still be read by earlier work on the stream
    if (moe_status st = moe::check_hip(hipStreamSynchronize(stream), "moe_slot_table_preload: sync")) return st;
  }
  bool changed = false;
  for (int i = 0; i < n; ++i) {
    const int l = layer_expert[2 * i], e = layer_expert[2 * i + 1];
    const int64_t idx = (int64_t)l * t->E + e;
    if (t->map[idx] >= 0) {
      lru_touch(t, t->map[idx]);
      continue;
    }
    const int s = place(t, l, e);
    if (moe_status st = do_copy(t, s, l, e, stream)) return st;
    changed = true;
  }
  return changed ? upload_map(t, stream) : MOE_OK;
}

moe_status moe_slot_table_resolve(moe_slot_table* t, int layer, const int32_t* active, const int32_t* n_active,
                                  hipStream_t stream) {
  if (!t || t->host_only) return fail(MOE_EINVAL, "moe_slot_table_resolve: not a device table");
  if (t->device_mode) return fail(MOE_EINVAL, "moe_slot_table_resolve: the table is in device mode");
  if (layer < 0 || layer >= t->L) return fail(MOE_EINVAL, "moe_slot_table_resolve: layer out of range");
  if (!active || !n_active) return fail(MOE_EINVAL, "moe_slot_table_resolve: null pointer");
  // 1) how many experts are active (waits for the routing work queued before us)
  if (moe_status st = moe::check_hip(hipMemcpyAsync(t->act_stage, n_active, sizeof(int32_t), hipMemcpyDeviceToHost,
                                                    stream), "moe_slot_table_resolve: copy n_active"))
    return st;
  if (moe_status st = moe::check_hip(hipStreamSynchronize(stream), "moe_slot_table_resolve: sync")) return st;
  const int n = t->act_stage[0];
  if (n < 0 || n > t->E) return fail(MOE_EINVAL, "moe_slot_table_resolve: n_active out of range");
  // 2) which
  if (n > 0) {
    if (moe_status st = moe::check_hip(hipMemcpyAsync(t->act_stage + 1, active, sizeof(int32_t) * (size_t)n,
                                                      hipMemcpyDeviceToHost, stream),
                                       "moe_slot_table_resolve: copy active"))
      return st;
    if (moe_status st = moe::check_hip(hipStreamSynchronize(stream), "moe_slot_table_resolve: sync")) return st;
  }
  bool changed = false;
  if (moe_status st = resolve_list(t, layer, t->act_stage + 1, n, stream, changed)) return st;
  return changed ? upload_map(t, stream) : MOE_OK;
}

moe_status moe_slot_table_resolve_host(moe_slot_table* t, int layer, const int32_t* active, int n_active) {
  if (!t || !t->host_only) return fail(MOE_EINVAL, "moe_slot_table_resolve_host: not a host-only table");
  if (layer < 0 || layer >= t->L) return fail(MOE_EINVAL, "moe_slot_table_resolve_host: layer out of range");
  if (n_active < 0 || (n_active > 0 && !active)) return fail(MOE_EINVAL, "moe_slot_table_resolve_host: bad list");
  bool changed = false;
  return resolve_list(t, layer, active, n_active, nullptr, changed);
}

moe_status moe_slot_table_stats(const moe_slot_table* t, moe_slot_stats* out) {
  if (!t || !out) return fail(MOE_EINVAL, "moe_slot_table_stats: null pointer");
  if (t->device_mode) {
    uint64_t v[5];
    if (moe_status st = moe::check_hip(hipMemcpy(v, t->d_stats, sizeof(v), hipMemcpyDeviceToHost),
                                       "moe_slot_table_stats: copy counters"))
      return st;
    *out = moe_slot_stats{v[0], v[1], v[2], v[3], v[4]};
    return MOE_OK;
  }
  *out = t->stats;
  return MOE_OK;
}

moe_status moe_slot_table_map_host(const moe_slot_table* t, int32_t* out) {
  if (!t || !out) return fail(MOE_EINVAL, "moe_slot_table_map_host: null pointer");
  if (t->device_mode)
    return moe::check_hip(hipMemcpy(out, t->slot_map_dev, t->map.size() * sizeof(int32_t), hipMemcpyDeviceToHost),
                          "moe_slot_table_map_host: copy map");
  std::memcpy(out, t->map.data(), t->map.size() * sizeof(int32_t));
  return MOE_OK;
}

size_t moe_slot_table_device_bytes(int L, int E, int n_slots) {
  if (L < 1 || E < 1 || E > moe::kMaxE || n_slots < 1) return 0;
  return dev_layout(E, n_slots).bytes;
}

moe_status moe_slot_table_enable_device(moe_slot_table* t, void* state, size_t state_bytes, hipStream_t stream) {
  if (!t || t->host_only) return fail(MOE_EINVAL, "moe_slot_table_enable_device: not a device table");
  if (t->device_mode) return fail(MOE_EINVAL, "moe_slot_table_enable_device: already in device mode");
  const DevLayout d = dev_layout(t->E, t->n_slots);
  if (!state || reinterpret_cast<uintptr_t>(state) % 256)
    return fail(MOE_EINVAL, "moe_slot_table_enable_device: state must be 256-byte aligned device memory");
  if (state_bytes < d.bytes)
    return fail(MOE_EWORKSPACE, "moe_slot_table_enable_device: state is " + std::to_string(state_bytes) +
                                    " bytes, needs " + std::to_string(d.bytes));
  void* hd = nullptr;
  if (moe_status st = moe::check_hip(hipHostGetDevicePointer(&hd, const_cast<uint8_t*>(t->host), 0),
                                     "moe_slot_table_enable_device: device mapping of the master copy"))
    return st;
  if (moe_status st = moe::check_hip(hipStreamSynchronize(stream), "moe_slot_table_enable_device: sync")) return st;
  // the host policy state in device form: stamps in LRU order (head = 0)
  std::vector<int64_t> stamp(t->n_slots, 0);
  int64_t clock = 0;
  for (int q = t->head; q >= 0; q = t->next[q]) stamp[q] = clock++;
  const uint64_t stats[5] = {t->stats.hits, t->stats.misses, t->stats.bytes_h2d, t->stats.resolves,
                             t->stats.evictions};
  uint8_t* b = static_cast<uint8_t*>(state);
  t->d_owner = reinterpret_cast<int32_t*>(b + d.owner);
  t->d_stamp = reinterpret_cast<int64_t*>(b + d.stamp);
  t->d_clock = reinterpret_cast<int64_t*>(b + d.clock);
  t->d_stats = reinterpret_cast<uint64_t*>(b + d.stats);
  t->d_copies = reinterpret_cast<int32_t*>(b + d.copies);
  t->d_ncopies = reinterpret_cast<int32_t*>(b + d.ncopies);
  t->d_ready = reinterpret_cast<uint64_t*>(b + d.ready);
  const int32_t zero = 0;
  const char* what = "moe_slot_table_enable_device: upload";
  if (moe_status st = moe::check_hip(hipMemcpy(t->d_owner, t->owner.data(), sizeof(int32_t) * t->n_slots,
                                               hipMemcpyHostToDevice), what))
    return st;
  if (moe_status st = moe::check_hip(hipMemcpy(t->d_stamp, stamp.data(), sizeof(int64_t) * t->n_slots,
                                               hipMemcpyHostToDevice), what))
    return st;
  if (moe_status st = moe::check_hip(hipMemcpy(t->d_clock, &clock, sizeof(clock), hipMemcpyHostToDevice), what))
    return st;
  if (moe_status st = moe::check_hip(hipMemcpy(t->d_stats, stats, sizeof(stats), hipMemcpyHostToDevice), what))
    return st;
  if (moe_status st = moe::check_hip(hipMemcpy(t->d_ncopies, &zero, sizeof(zero), hipMemcpyHostToDevice), what))
    return st;
  // the ready word of the in-launch resolve: never clock + 1 for a clock yet to come
  const uint64_t ready = (uint64_t)clock;
  if (moe_status st = moe::check_hip(hipMemcpy(t->d_ready, &ready, sizeof(ready), hipMemcpyHostToDevice), what))
    return st;
  t->host_dev = static_cast<const uint8_t*>(hd);
  t->device_mode = true;
  return MOE_OK;
}

moe_status moe_slot_table_resolve_device(moe_slot_table* t, int layer, const int32_t* active,
                                         const int32_t* n_active, int max_active, hipStream_t stream) {
  if (!t || !t->device_mode) return fail(MOE_EINVAL, "moe_slot_table_resolve_device: table not in device mode");
  if (layer < 0 || layer >= t->L) return fail(MOE_EINVAL, "moe_slot_table_resolve_device: layer out of range");
  if (!active || !n_active) return fail(MOE_EINVAL, "moe_slot_table_resolve_device: null pointer");
  if (max_active < 1 || max_active > t->E)
    return fail(MOE_EINVAL, "moe_slot_table_resolve_device: max_active outside [1, E]");
  if (max_active > t->n_slots)
    return fail(MOE_ECAPACITY, "moe_slot_table_resolve_device: up to " + std::to_string(max_active) +
                                   " active experts, " + std::to_string(t->n_slots) + " slots");
  slot_resolve_kernel<<<1, kResolveThreads, 0, stream>>>(moe::slot_dev_args(t), layer, active, n_active, max_active);
  if (moe_status st = moe::check_launch("slot_resolve")) return st;
  return moe::launch_slot_copy(t, stream);
}

void moe_slot_table_destroy(moe_slot_table* t) { free_table(t); }

}  // extern "C"

namespace moe {

bool slot_table_device_mode(const moe_slot_table* t) { return t && t->device_mode; }

SlotDevArgs slot_dev_args(const moe_slot_table* t) {
  SlotDevArgs a;
  a.map = t->slot_map_dev;
  a.owner = t->d_owner;
  a.stamp = t->d_stamp;
  a.clock = t->d_clock;
  a.stats = t->d_stats;
  a.copies = t->d_copies;
  a.ncopies = t->d_ncopies;
  a.ready = t->d_ready;
  a.E = t->E;
  a.n_slots = t->n_slots;
  a.expert_bytes = t->expert_bytes;
  return a;
}

SlotTableView slot_table_view(const moe_slot_table* t) {
  return SlotTableView{t->L,      t->E,        t->n_slots,  t->expert_bytes, t->slots,
                       t->slot_map_dev, t->host_dev, t->d_copies, t->d_ncopies};
}

moe_status launch_slot_copy(const moe_slot_table* t, hipStream_t stream) {
  slot_copy_kernel<<<kCopyGrid, kCopyThreads, 0, stream>>>(t->d_copies, t->d_ncopies, t->host_dev, t->slots,
                                                            (int64_t)t->expert_bytes);
  return check_launch("slot_copy");
}

}  // namespace moe
