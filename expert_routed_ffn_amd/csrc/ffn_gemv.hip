// ffn_gemv.hip -- expert FFN for decode and verify steps (few tokens per expert).
//
// Passage: only the routed experts' weights are touched per token (Strata
// feature, tech.hub77a.com, summary row "핵심 기법" and section "2. 왜 대단한가"
// (1)); verify steps run 1 + d tokens through the model at once (same page,
// (3)); the fast size is a 2-bit class quantization (section "3. 바로 써먹기").
//
// For each active expert e and each of its n_e routed rows x:
//   g = Wg x, u = Wu x, h = silu(g) * u    (h kept to about 16 significant bits)
//   y = Wd h                               (written per assignment)
//
// Arithmetic per block of 32 weights (scale s, min m, codes q):
//   sum_c (s*q_c + m) x_c = s * sum_c (128 + q_c) x_c + (m - 128*s) * sum_c x_c.
// (128 + q) is a bf16 whose bit pattern is 0x4300 | q, so two codes become a
// packed bf16 pair with one shift and one and-or (the code layout puts
// adjacent columns in the two halfwords of a word; 3-bit codes or in their high
// bits from the block's third word), and v_dot2c_f32_bf16 does the two MACs
// against the packed input pair with fp32 accumulation.
// sum_c x_c is per input row and chunk, computed once per wave.  Inputs that
// are not bf16 (fp32 activations, h) are carried as an unevaluated sum
// hi + lo of two bf16 values (about 16 significant bits), so the products
// stay exact and accumulation is fp32.
//
// Work split.  A row of K weights is cut into K/32 chunks (one scale/min block
// each).  G lanes share a row, each owning K/(32G) chunks; lane partial sums
// are reduced across the G lanes.
//
// Two kernel families:
//  * wide (H a multiple of 2048 and I a multiple of 512, the shapes of the
//    decode workloads).  Gate/up: one workgroup per (active expert, tile of
//    I); a row is split over all 64 lanes of a wave, so a lane's activation
//    chunk stays in registers for all its rows; activation loads are issued
//    before the weight loads and rows are consumed in load order; the lane
//    partials of all (row, token) pairs are reduced together by a
//    reduce-scatter (each exchange level halves the values a lane carries:
//    permlane32/16 swaps, then DPP), about two instructions per value instead
//    of two per value and level; h is written as separate bf16 hi and lo
//    planes.  Down: row-tiled, one workgroup per 8 output rows over every
//    routed row (16 lanes per row), so the layer's combine can be folded into
//    the same launch (each workgroup owns all contributions to its rows).
//  * general (any H, I that are multiples of 32): G = gcd(K/32, 64) lanes per
//    row, a butterfly reduction per (row, token), h in fp32, one workgroup per
//    (active expert, row tile) for both products.
//
// Scheduling.  A decode step moves ~20 MB, a few microseconds of HBM time, so
// launch and dependency latency dominate.  In the layer step (wide shapes) the
// gate/up workgroups route the tokens themselves from the logits (a few KB
// every workgroup reads through the L2) instead of waiting for a routing
// launch; one extra workgroup writes the routing and dispatch outputs,
// including a per-position (expert, assignment) table the down kernel reads
// after the launch boundary.  Called on its own, the gate/up kernel reads a
// per-expert descriptor (id, first row, row count, tokens) built by a small
// preceding kernel, one dependent load.
#include "internal.hpp"
#include "route_dispatch_dev.hpp"
#include "slot_dev.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// f = hi + lo with hi, lo bf16: packed hi pairs and lo pairs of (a, b).
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - bf16lo(hi), b - bf16hi(hi));
}

// One 32-column chunk of an input row: 16 packed pairs (hi, and lo when split)
// and the chunk sum.
template <bool SPLIT>
struct XChunk {
  uint32_t hi[16];
  uint32_t lo[SPLIT ? 16 : 1];
  float sum;
};

__device__ __forceinline__ void load_chunk(XChunk<false>& c, const uint16_t* p /* 32 bf16, 16-byte aligned */) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = q[i];
    c.hi[4 * i + 0] = v.x;
    c.hi[4 * i + 1] = v.y;
    c.hi[4 * i + 2] = v.z;
    c.hi[4 * i + 3] = v.w;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s = dot2(c.hi[i], 0x3F803F80u, s);  // x_even + x_odd, fp32
  c.sum = s;
}

__device__ __forceinline__ void load_chunk(XChunk<true>& c, const float* p /* 32 floats, 16-byte aligned */) {
  const float4* q = reinterpret_cast<const float4*>(p);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = q[i];
    split_pair(v.x, v.y, c.hi[2 * i], c.lo[2 * i]);
    split_pair(v.z, v.w, c.hi[2 * i + 1], c.lo[2 * i + 1]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s = dot2(c.hi[i], 0x3F803F80u, s);
    s = dot2(c.lo[i], 0x3F803F80u, s);
  }
  c.sum = s;
}

// (x & m) | c in one VALU op.  gfx950's three-operand encoding takes no
// literal constants, so the compiler otherwise splits this into an and plus
// an or; m lives in a scalar register, c in a vector register.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

// sum over the chunk of (128 + q_c) * x_c for the BITS-bit codes in `code`.
template <int BITS, bool SPLIT>
__device__ __forceinline__ float chunk_dot(const uint32_t (&code)[BITS], const XChunk<SPLIT>& x) {
  float acc = 0.f;
  if constexpr (BITS == 3) {
    // words 0-1: the low two bits of the pairs as in the 2-bit layout; word 2:
    // the high bit of column pair P at bits P and 16 + P
#pragma unroll
    for (int P = 0; P < 16; ++P) {
      const uint32_t hi = (code[2] >> P) & 0x00010001u;
      const uint32_t v = and_or(code[P / 8] >> (2 * (P % 8)), 0x00030003u, 0x43004300u) | (hi << 2);
      acc = dot2(v, x.hi[P], acc);
      if constexpr (SPLIT) acc = dot2(v, x.lo[P], acc);
    }
    return acc;
  }
  constexpr uint32_t kMask = BITS == 2 ? 0x00030003u : 0x000F000Fu;
  constexpr int kPairs = 16 / BITS;  // code pairs per word
#pragma unroll
  for (int d = 0; d < BITS; ++d)
#pragma unroll
    for (int p = 0; p < kPairs; ++p) {
      const uint32_t v = and_or(code[d] >> (BITS * p), kMask, 0x43004300u);
      acc = dot2(v, x.hi[d * kPairs + p], acc);
      if constexpr (SPLIT) acc = dot2(v, x.lo[d * kPairs + p], acc);
    }
  return acc;
}

// Weight codes, and the gate and up scale/min words, are loaded as streaming
// (nontemporal) accesses: a decode step reads each of them once (a down
// workgroup reads the codes of an expert's several positions back to back),
// and they then do not displace the activations, h and routing data that the
// workgroups re-read from the L2.  Decode/verify layer step 19.46 -> 18.34 us
// on one box.  The down scale/min words (two rows per cache line, read by
// different lane groups) measured slower that way (18.9 us) and keep ordinary
// loads.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT = false>
__device__ __forceinline__ uint32_t load_sm(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  return *reinterpret_cast<const uint32_t*>(p);
}

template <int BITS, bool NT = false>
__device__ __forceinline__ void load_codes(uint32_t (&code)[BITS], const uint8_t* p) {
  if constexpr (BITS == 2) {
    const u32x2_t* q = reinterpret_cast<const u32x2_t*>(p);
    u32x2_t v;
    if constexpr (NT) v = __builtin_nontemporal_load(q);
    else v = *q;
    code[0] = v.x;
    code[1] = v.y;
  } else if constexpr (BITS == 3) {  // 12-byte chunks: 4-byte aligned only
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if constexpr (NT) code[i] = __builtin_nontemporal_load(q + i);
      else code[i] = q[i];
    }
  } else {
    const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
    u32x4_t v;
    if constexpr (NT) v = __builtin_nontemporal_load(q);
    else v = *q;
    code[0] = v.x;
    code[1] = v.y;
    code[2] = v.z;
    code[3] = v.w;
  }
}

// Writes back what load_codes read, as a buffer store at lane offset `lo`
// plus the wave-uniform offset `so` of a resource over the destination blob
// (no 64-bit address registers held for it).
template <int BITS>
__device__ __forceinline__ void store_codes_buf(__amdgpu_buffer_rsrc_t rd, uint32_t lo, uint32_t so,
                                                const uint32_t (&code)[BITS]) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  so = __builtin_amdgcn_readfirstlane(so);
  if constexpr (BITS == 2) __builtin_amdgcn_raw_buffer_store_b64(u32x2{code[0], code[1]}, rd, lo, so, 0);
  else if constexpr (BITS == 3) __builtin_amdgcn_raw_buffer_store_b96(u32x3{code[0], code[1], code[2]}, rd, lo, so, 0);
  else __builtin_amdgcn_raw_buffer_store_b128(u32x4{code[0], code[1], code[2], code[3]}, rd, lo, so, 0);
}

__device__ __forceinline__ float group_sum(float v, int G) {
  for (int off = 1; off < G; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

struct Geo {
  int G;    // lanes per row (power of two dividing 64)
  int CPL;  // chunks per lane = (K / 32) / G
};

inline int gcd_pow2_64(int nc) {
  int g = 1;
  while (g < 64 && nc % (2 * g) == 0) g *= 2;
  return g;
}

// Rows per lane by the largest number of routed rows a pass handles (TM).
// Measured on the decode/verify workload: a wave's time grows by roughly one
// memory round trip per extra row, so few rows per wave and many waves win
// (gate/up 14.3 us at 2 rows, 15.8 at 4, 23.9 at 8; down 15.6 us at 4 rows).
#ifndef MOE_RL_GU_1
#define MOE_RL_GU_1 4
#endif
#ifndef MOE_RL_GU_3
#define MOE_RL_GU_3 2
#endif
#ifndef MOE_RL_GU_4
#define MOE_RL_GU_4 2
#endif
#ifndef MOE_RL_DN_1
#define MOE_RL_DN_1 8
#endif
#ifndef MOE_RL_DN_3
#define MOE_RL_DN_3 4
#endif
#ifndef MOE_RL_DN_4
#define MOE_RL_DN_4 4
#endif
template <int TM> constexpr int kRLGateUp = TM >= 4 ? MOE_RL_GU_4 : TM == 3 ? MOE_RL_GU_3 : MOE_RL_GU_1;
template <int TM> constexpr int kRLGateUpSplit = TM >= 3 ? 4 : 8;
template <int TM> constexpr int kRLDown = TM >= 4 ? MOE_RL_DN_4 : TM == 3 ? MOE_RL_DN_3 : MOE_RL_DN_1;

// Brings every 64-byte line of the first BYTES bytes of the kernel-argument
// segment into the scalar cache with one round trip.  The decode kernels' large
// argument structs and their scalar register pressure make the compiler load
// arguments where they are first used and wait after each load, so a workgroup
// otherwise pays several dependent cache misses before its first memory access.
// The words read are discarded; every read lies inside the segment.
#ifndef MOE_WARM_KERNARGS
#define MOE_WARM_KERNARGS 1
#endif
template <int BYTES>
__device__ __forceinline__ void warm_kernargs() {
  if constexpr (MOE_WARM_KERNARGS != 0) {
    typedef __attribute__((address_space(4))) const uint32_t kword_t;
    kword_t* k = (kword_t*)__builtin_amdgcn_kernarg_segment_ptr();
    uint32_t d = 0;
#pragma unroll
    for (int off = 64; off + 4 <= BYTES; off += 64) d ^= k[off / 4];
    asm volatile("" ::"s"(d));
  }
}

struct DecodeArgs {
  const uint8_t* base;
  int64_t stride;
  const int32_t* slot_map;
  int H, I, k, T;
  int64_t off_gc, off_gs, off_uc, off_us, off_dc, off_ds;
  const void* xin;
  const int32_t* n_active;
  const SlotDesc* desc;
  const int32_t* sorted_assign;
  float* h;       // general kernels: fp32 h [T*k x I]
  uint16_t* hh;   // wide kernels: bf16 hi plane of h [T*k x I] ...
  uint16_t* hl;   // ... and lo plane (same bytes as the fp32 h)
  void* y;
  const int32_t* rows;   // (expert, assignment) per sorted position
  const int32_t* nrows;  // number of sorted positions
  const int32_t* pos_slot;  // NULL, or the slot of each sorted position (overrides slot_map in the down rows)
  // combine folded into the row-tiled down kernel (out == nullptr: not folded)
  const float* w;
  const void* residual;
  int r_bf16;
  float* out;
  uint16_t* out_bf16;
  int E;
  int TA, TB;  // gate/up and down workgroups per expert
  Geo ga, gb;
};

// One active expert as an item sees it: scalars plus the descriptor in memory
// (its token lists are read through the pointer, never copied into an
// indexed local array).
struct Slot {
  const SlotDesc* p;
  int e, p0, ne;
  int tokv;  // wide kernels: lane j < kDescT holds the token of row j
};

__device__ __forceinline__ Slot load_slot(const DecodeArgs& A, int s) {
  const SlotDesc* p = A.desc + s;
  return Slot{p, p->e, p->p0, p->ne, 0};
}

// Token and assignment of the rel-th routed row of a slot.
__device__ __forceinline__ int row_token(const DecodeArgs& A, const Slot& d, int rel) {
  return rel < kDescT ? d.p->tok[rel] : A.sorted_assign[d.p0 + rel] / A.k;
}
__device__ __forceinline__ int row_token_w(const DecodeArgs& A, const Slot& d, int rel) {
  return rel < kDescT ? __builtin_amdgcn_readlane(d.tokv, rel) : A.sorted_assign[d.p0 + rel] / A.k;
}
__device__ __forceinline__ int row_assign(const DecodeArgs& A, const Slot& d, int rel) {
  return rel < kDescT ? d.p->asg[rel] : A.sorted_assign[d.p0 + rel];
}

__device__ __forceinline__ int resident_index(const DecodeArgs& A, int e) { return A.slot_map ? A.slot_map[e] : e; }

// ---- gate/up ----------------------------------------------------------------
// One pass over the wave's rows for the NT routed rows rel0 .. rel0+NT-1.
template <int BITS, int NT, bool SPLIT, int RL>
__device__ __forceinline__ void gateup_pass(const DecodeArgs& A, const Slot& d, const uint8_t* blob, int i0,
                                            int rel0) {
  const int lane = threadIdx.x & 63;
  const int G = A.ga.G, RPI = 64 / G, sl = lane / G, gl = lane % G;
  const int NI = RL * RPI / 2;
  const int64_t row_code_bytes = (int64_t)A.H * BITS / 8, row_sm_bytes = (int64_t)(A.H / 32) * 4;
  int64_t tok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) tok[t] = row_token(A, d, rel0 + t);

  float part[RL][NT];
#pragma unroll
  for (int r = 0; r < RL; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) part[r][t] = 0.f;

  for (int cc = 0; cc < A.ga.CPL; ++cc) {
    const int chunk = gl + G * cc;
    uint32_t code[RL][BITS];
    uint32_t smw[RL];
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      const int rho = r * RPI + sl;
      const bool up = rho >= NI;
      int i = i0 + (up ? rho - NI : rho);
      i = i < A.I ? i : A.I - 1;  // rows past I are computed on a valid row and dropped
      load_codes<BITS, true>(code[r], blob + (up ? A.off_uc : A.off_gc) + i * row_code_bytes + chunk * (4 * BITS));
      smw[r] = load_sm<true>(blob + (up ? A.off_us : A.off_gs) + i * row_sm_bytes + chunk * 4);
    }
    XChunk<SPLIT> xc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (SPLIT)
        load_chunk(xc[t], reinterpret_cast<const float*>(A.xin) + tok[t] * A.H + 32 * chunk);
      else
        load_chunk(xc[t], reinterpret_cast<const uint16_t*>(A.xin) + tok[t] * A.H + 32 * chunk);
    }
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      const float s = f16lo(smw[r]), m = f16hi(smw[r]);
      const float mo = m - 128.0f * s;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        part[r][t] = __builtin_fmaf(s, chunk_dot<BITS, SPLIT>(code[r], xc[t]), __builtin_fmaf(mo, xc[t].sum, part[r][t]));
    }
  }

#pragma unroll
  for (int r = 0; r < RL; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) part[r][t] = group_sum(part[r][t], G);

  if (gl == 0) {
#pragma unroll
    for (int r = 0; r < RL / 2; ++r) {
      const int i = i0 + r * RPI + sl;
      if (i >= A.I) continue;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float g = part[r][t], u = part[r + RL / 2][t];
        A.h[(size_t)(d.p0 + rel0 + t) * A.I + i] = g / (1.0f + expf(-g)) * u;
      }
    }
  }
}

template <int BITS, int TM, bool SPLIT, int RL>
__device__ __forceinline__ void item_gateup(const DecodeArgs& A, const Slot& d, int j) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = A.ga.G, RPI = 64 / G, sl = lane / G, gl = lane % G;
  const int NI = RL * RPI / 2;
  const int i0 = (j * 4 + wave) * NI;
  if (i0 >= A.I) return;
  const int idx = resident_index(A, d.e);
  if (idx < 0) {  // expert not resident: poison its h rows
    for (int r = 0; r < RL / 2; ++r) {
      const int i = i0 + r * RPI + sl;
      if (gl == 0 && i < A.I)
        for (int t = 0; t < d.ne; ++t) A.h[(size_t)(d.p0 + t) * A.I + i] = __builtin_nanf("");
    }
    return;
  }
  const uint8_t* blob = A.base + (int64_t)idx * A.stride;
  for (int tg = 0; tg < d.ne;) {
    const int nt = min(d.ne - tg, TM);
    if (nt >= 4) gateup_pass<BITS, (TM >= 4 ? 4 : 1), SPLIT, RL>(A, d, blob, i0, tg);
    else if (nt == 3) gateup_pass<BITS, (TM >= 3 ? 3 : 1), SPLIT, RL>(A, d, blob, i0, tg);
    else if (nt == 2) gateup_pass<BITS, (TM >= 2 ? 2 : 1), SPLIT, RL>(A, d, blob, i0, tg);
    else gateup_pass<BITS, 1, SPLIT, RL>(A, d, blob, i0, tg);
    tg += nt;
  }
}

// ---- down (general) -------------------------------------------------------------
template <int BITS, int RL>
struct DownPre {
  uint32_t code[RL][BITS];
  uint32_t smw[RL];
};

template <int BITS, int RL>
__device__ __forceinline__ void down_load(const DecodeArgs& A, const uint8_t* blob, int n0, int cc,
                                          DownPre<BITS, RL>& P) {
  const int lane = threadIdx.x & 63;
  const int G = A.gb.G, RPI = 64 / G, sl = lane / G, gl = lane % G;
  const int64_t row_code_bytes = (int64_t)A.I * BITS / 8, row_sm_bytes = (int64_t)(A.I / 32) * 4;
  const int chunk = gl + G * cc;
#pragma unroll
  for (int r = 0; r < RL; ++r) {
    int n = n0 + r * RPI + sl;
    n = n < A.H ? n : A.H - 1;
    load_codes<BITS, true>(P.code[r], blob + A.off_dc + n * row_code_bytes + chunk * (4 * BITS));
    P.smw[r] = load_sm(blob + A.off_ds + n * row_sm_bytes + chunk * 4);
  }
}

// Accumulate one chunk (cc) of the down rows for NT routed rows.
template <int BITS, int NT, int RL>
__device__ __forceinline__ void down_chunk(const DecodeArgs& A, const Slot& d, int rel0, int cc,
                                           const DownPre<BITS, RL>& P, float (&part)[RL][NT]) {
  const int lane = threadIdx.x & 63;
  const int G = A.gb.G, gl = lane % G;
  const int chunk = gl + G * cc;
  XChunk<true> hc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) load_chunk(hc[t], A.h + (size_t)(d.p0 + rel0 + t) * A.I + 32 * chunk);
#pragma unroll
  for (int r = 0; r < RL; ++r) {
    const float s = f16lo(P.smw[r]), m = f16hi(P.smw[r]);
    const float mo = m - 128.0f * s;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      part[r][t] = __builtin_fmaf(s, chunk_dot<BITS, true>(P.code[r], hc[t]), __builtin_fmaf(mo, hc[t].sum, part[r][t]));
  }
}

template <int BITS, int NT, int RL, bool YBF16>
__device__ __forceinline__ void down_pass(const DecodeArgs& A, const Slot& d, const uint8_t* blob, int n0,
                                          int rel0, bool resident) {
  const int lane = threadIdx.x & 63;
  const int G = A.gb.G, RPI = 64 / G, sl = lane / G, gl = lane % G;
  float part[RL][NT];
#pragma unroll
  for (int r = 0; r < RL; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) part[r][t] = 0.f;

  if (resident) {
    for (int cc = 0; cc < A.gb.CPL; ++cc) {
      DownPre<BITS, RL> P;
      down_load<BITS, RL>(A, blob, n0, cc, P);
      down_chunk<BITS, NT, RL>(A, d, rel0, cc, P, part);
    }
  }

#pragma unroll
  for (int r = 0; r < RL; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) part[r][t] = group_sum(part[r][t], G);

  if (gl == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t a = row_assign(A, d, rel0 + t);
#pragma unroll
      for (int r = 0; r < RL; ++r) {
        const int n = n0 + r * RPI + sl;
        if (n >= A.H) continue;
        const float v = resident ? part[r][t] : __builtin_nanf("");
        if constexpr (YBF16) reinterpret_cast<uint16_t*>(A.y)[a * A.H + n] = __builtin_bit_cast(uint16_t, (__bf16)v);
        else reinterpret_cast<float*>(A.y)[a * A.H + n] = v;
      }
    }
  }
}

template <int BITS, int TM, int RL, bool YBF16>
__device__ __forceinline__ void item_down(const DecodeArgs& A, const Slot& d, int j) {
  const int wave = threadIdx.x >> 6;
  const int RPI = 64 / A.gb.G;
  const int n0 = (j * 4 + wave) * RL * RPI;
  if (n0 >= A.H) return;
  const int idx = resident_index(A, d.e);
  const bool resident = idx >= 0;
  const uint8_t* blob = A.base + (int64_t)(resident ? idx : 0) * A.stride;
  for (int tg = 0; tg < d.ne;) {
    const int nt = min(d.ne - tg, TM);
    if (nt >= 4) down_pass<BITS, (TM >= 4 ? 4 : 1), RL, YBF16>(A, d, blob, n0, tg, resident);
    else if (nt == 3) down_pass<BITS, (TM >= 3 ? 3 : 1), RL, YBF16>(A, d, blob, n0, tg, resident);
    else if (nt == 2) down_pass<BITS, (TM >= 2 ? 2 : 1), RL, YBF16>(A, d, blob, n0, tg, resident);
    else down_pass<BITS, 1, RL, YBF16>(A, d, blob, n0, tg, resident);
    tg += nt;
  }
}

// ---- cross-lane reduce-scatter (wave64) --------------------------------------------
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// One exchange level over lane bit BIT.  Lanes with the bit clear return
// a + a(partner), lanes with the bit set return b + b(partner); the partner
// differs in that bit.  Bit 5: v_permlane32_swap (swaps the upper half of one
// register with the lower half of the other), bit 4: v_permlane16_swap (odd
// 16-lane rows with even ones); bits 3..0 stay inside a 16-lane row: DPP
// row_ror:8 (lane i <-> i^8), row_half_mirror (i <-> 7-i within 8, which
// differs from i in bit 2), quad_perm [2,3,0,1] and [1,0,3,2].
template <int BIT>
__device__ __forceinline__ float scatter_pair(float a, float b, int lane) {
  if constexpr (BIT == 5 || BIT == 4) {
    const u32x2_t r = BIT == 5 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                               : __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r.x) + __uint_as_float(r.y);
  } else {
    constexpr int kCtrl = BIT == 3 ? 0x128 : BIT == 2 ? 0x141 : BIT == 1 ? 0x4E : 0xB1;
    const bool hi = (lane >> BIT) & 1;
    const float send = hi ? a : b, keep = hi ? b : a;
    return keep + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), kCtrl, 0xF, 0xF, false));
  }
}

// v + v(partner over lane bit BIT): both lanes of a pair end with the sum.
template <int BIT>
__device__ __forceinline__ float butterfly(float v) {
  if constexpr (BIT == 5 || BIT == 4) {
    const uint32_t u = __float_as_uint(v);
    const u32x2_t r = BIT == 5 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                               : __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r.x) + __uint_as_float(r.y);
  } else {
    constexpr int kCtrl = BIT == 3 ? 0x128 : BIT == 2 ? 0x141 : BIT == 1 ? 0x4E : 0xB1;
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
  }
}

// Sums v[0..NV) over the lanes that differ in bits BIT..BOT.  While a lane
// carries more than KEEP values, each level keeps one half (the first half
// where the lane's bit is clear); after the last such level the remaining
// levels are butterflies.  On return v[0..NVf) holds sums, NVf = NV >> S for
// S = min(log2(NV / KEEP), BIT - BOT + 1) halving levels, and v[i] is value
// number blk * NVf + i, blk being the lane's bits BIT .. BIT-S+1 read as a
// binary number (BIT the most significant).
template <int NV, int KEEP, int BIT, int BOT>
__device__ __forceinline__ void reduce_scatter(float* v, int lane) {
  if constexpr (BIT >= BOT) {
    if constexpr (NV > KEEP) {
#pragma unroll
      for (int i = 0; i < NV / 2; ++i) v[i] = scatter_pair<BIT>(v[i], v[i + NV / 2], lane);
      reduce_scatter<NV / 2, KEEP, BIT - 1, BOT>(v, lane);
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i] = butterfly<BIT>(v[i]);
      reduce_scatter<NV, KEEP, BIT - 1, BOT>(v, lane);
    }
  }
}

constexpr int pow2_ceil(int v) { return v <= 1 ? 1 : 2 * pow2_ceil((v + 1) / 2); }
constexpr int log2_exact(int v) { return v <= 1 ? 0 : 1 + log2_exact(v / 2); }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

// ---- wide kernels: gate/up over 64 lanes, down over 16 lanes ------------------------
// Raw activation chunk (32 columns) of one token: bf16 (16 packed pairs) or
// fp32 (32 floats, split later).
template <bool SPLIT>
struct RawX {
  uint32_t w[SPLIT ? 32 : 16];
};

template <bool SPLIT>
__device__ __forceinline__ void load_raw(RawX<SPLIT>& r, const void* xin, int64_t tok, int H, int chunk) {
  const uint4* q = SPLIT ? reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(xin) + tok * H + 32 * chunk)
                         : reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(xin) + tok * H + 32 * chunk);
#pragma unroll
  for (int i = 0; i < (SPLIT ? 8 : 4); ++i) {
    const uint4 v = q[i];
    r.w[4 * i + 0] = v.x;
    r.w[4 * i + 1] = v.y;
    r.w[4 * i + 2] = v.z;
    r.w[4 * i + 3] = v.w;
  }
}

// Same packed pairs and chunk sum as load_chunk, from registers.
template <bool SPLIT>
__device__ __forceinline__ void make_chunk(XChunk<SPLIT>& c, const RawX<SPLIT>& r) {
  float s = 0.f;
  if constexpr (SPLIT) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      split_pair(__uint_as_float(r.w[2 * i]), __uint_as_float(r.w[2 * i + 1]), c.hi[i], c.lo[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s = dot2(c.hi[i], 0x3F803F80u, s);
      s = dot2(c.lo[i], 0x3F803F80u, s);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) c.hi[i] = r.w[i];
#pragma unroll
    for (int i = 0; i < 16; ++i) s = dot2(c.hi[i], 0x3F803F80u, s);
  }
  c.sum = s;
}

// I rows (gate and up) per wave of the wide gate/up kernel.
#ifndef MOE_WIDE_NI
#define MOE_WIDE_NI 4
#endif
#ifndef MOE_WIDE_NI_SPLIT
#define MOE_WIDE_NI_SPLIT 2
#endif
constexpr int kWideTM = 3;  // routed rows per pass in the wide gate/up kernel
template <bool SPLIT> constexpr int kWideNI = SPLIT ? MOE_WIDE_NI_SPLIT : MOE_WIDE_NI;

// STAGE: when dst is set, blob is a missed expert's master copy and the pass
// also writes every code and s/m word it reads to the same offsets of dst,
// the expert's slot.
template <int BITS, int NT, bool SPLIT, int NI, bool STAGE = false>
__device__ __forceinline__ void gateup_pass_wide(const DecodeArgs& A, const Slot& d, const uint8_t* blob, int i0,
                                                 int rel0, uint8_t* dst = nullptr) {
  const int lane = threadIdx.x & 63;
  const int64_t rcb = (int64_t)A.H * BITS / 8, rsb = (int64_t)(A.H / 32) * 4;
  int64_t tok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) tok[t] = row_token_w(A, d, rel0 + t);
  int64_t ri[NI];
#pragma unroll
  for (int r = 0; r < NI; ++r) ri[r] = min(i0 + r, A.I - 1);  // rows past I compute on a valid row, dropped

  float pg[NI][NT], pu[NI][NT];
#pragma unroll
  for (int r = 0; r < NI; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) pg[r][t] = pu[r][t] = 0.f;

  const int cpl = A.H / 2048;
  for (int cc = 0; cc < cpl; ++cc) {
    const int chunk = lane + 64 * cc;
    RawX<SPLIT> rx[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) load_raw<SPLIT>(rx[t], A.xin, tok[t], A.H, chunk);
    uint32_t cg[NI][BITS], cu[NI][BITS], sg[NI], su[NI];
#pragma unroll
    for (int r = 0; r < NI; ++r) {
      load_codes<BITS, true>(cg[r], blob + A.off_gc + ri[r] * rcb + chunk * (4 * BITS));
      sg[r] = load_sm<true>(blob + A.off_gs + ri[r] * rsb + chunk * 4);
      load_codes<BITS, true>(cu[r], blob + A.off_uc + ri[r] * rcb + chunk * (4 * BITS));
      su[r] = load_sm<true>(blob + A.off_us + ri[r] * rsb + chunk * 4);
    }
    if constexpr (STAGE) {
      // Buffer stores through a resource over dst; without dst the resource
      // has no records and the hardware drops every store (no branch, no
      // traffic).  Offsets fit in 32 bits: an expert blob is far below 4 GiB.
      // Rows past I repeat row I - 1 and rewrite its bytes unchanged.
      const __amdgpu_buffer_rsrc_t rd =
          __builtin_amdgcn_make_buffer_rsrc(dst ? dst : const_cast<uint8_t*>(blob), (short)0, dst ? -1 : 0, 0x00020000);
      const uint32_t lc = (uint32_t)(chunk * (4 * BITS)), ls = (uint32_t)(chunk * 4);
#pragma unroll
      for (int r = 0; r < NI; ++r) {
        store_codes_buf<BITS>(rd, lc, (uint32_t)(A.off_gc + ri[r] * rcb), cg[r]);
        __builtin_amdgcn_raw_buffer_store_b32(sg[r], rd, ls,
                                              __builtin_amdgcn_readfirstlane((uint32_t)(A.off_gs + ri[r] * rsb)), 0);
        store_codes_buf<BITS>(rd, lc, (uint32_t)(A.off_uc + ri[r] * rcb), cu[r]);
        __builtin_amdgcn_raw_buffer_store_b32(su[r], rd, ls,
                                              __builtin_amdgcn_readfirstlane((uint32_t)(A.off_us + ri[r] * rsb)), 0);
      }
    }
    XChunk<SPLIT> xc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) make_chunk<SPLIT>(xc[t], rx[t]);
#pragma unroll
    for (int r = 0; r < NI; ++r) {
      const float s1 = f16lo(sg[r]), m1 = f16hi(sg[r]), s2 = f16lo(su[r]), m2 = f16hi(su[r]);
      const float mo1 = m1 - 128.0f * s1, mo2 = m2 - 128.0f * s2;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        pg[r][t] = __builtin_fmaf(s1, chunk_dot<BITS, SPLIT>(cg[r], xc[t]), __builtin_fmaf(mo1, xc[t].sum, pg[r][t]));
        pu[r][t] = __builtin_fmaf(s2, chunk_dot<BITS, SPLIT>(cu[r], xc[t]), __builtin_fmaf(mo2, xc[t].sum, pu[r][t]));
      }
    }
  }

  // value 2m + {0: gate, 1: up} for m = r * NT + t, padded to a power of two
  constexpr int M = NI * NT, MP = pow2_ceil(M), S = log2_exact(MP);
  static_assert(S <= 6, "at most 64 (row, token) pairs per wave");
  float v[2 * MP];
#pragma unroll
  for (int m = 0; m < MP; ++m) {
    v[2 * m] = m < M ? pg[m / NT][m % NT] : 0.f;
    v[2 * m + 1] = m < M ? pu[m / NT][m % NT] : 0.f;
  }
  reduce_scatter<2 * MP, 2, 5, 0>(v, lane);
  const int m = lane >> (6 - S);
  if ((lane & ((1 << (6 - S)) - 1)) == 0 && m < M) {
    const int r = m / NT, t = m % NT, i = i0 + r;
    if (i < A.I) {
      const float g = v[0], u = v[1];
      const float hv = g / (1.0f + expf(-g)) * u;
      const size_t o = (size_t)(d.p0 + rel0 + t) * A.I + i;
      const __bf16 hb = (__bf16)hv;
      A.hh[o] = __builtin_bit_cast(uint16_t, hb);
      A.hl[o] = __builtin_bit_cast(uint16_t, (__bf16)(hv - (float)hb));
    }
  }
}

// Misses of a device-mode resolve staged by the gate/up launch (MissStage on
// the host side).  The first ncw workgroups of the grid copy the bytes of each
// missed blob that no gate/up item writes: everything outside the gate and up
// code and s/m planes, i.e. the down planes and the padding between planes.
struct StageArgs {
  const int32_t* copies;   // [2 * n] (slot, l*E + e)
  const int32_t* ncopies;  // [1] n
  const uint8_t* host;     // device view of the master copy, blob l*E + e at (l*E + e) * stride
  int64_t item_lo[4], item_hi[4];  // byte ranges [lo, hi) of the blob the gate/up items write
  int ncw;                 // copy workgroups at the front of the grid
};

// The master blob of slot `idx` if this step's resolve listed it as a miss,
// else null.  Wave-uniform.
__device__ __forceinline__ const uint8_t* staged_source(const StageArgs& G, int64_t stride, int idx) {
  const int lane = threadIdx.x & 63, nc = *G.ncopies;
  for (int c0 = 0; c0 < nc; c0 += 64) {
    const int c = c0 + lane;
    const uint64_t m = __ballot(c < nc && G.copies[2 * c] == idx);
    if (m) return G.host + (int64_t)G.copies[2 * (c0 + __builtin_ctzll(m)) + 1] * stride;
  }
  return nullptr;
}

// The passes of one gate/up item over its expert's routed rows, reading blob;
// with STAGE and dst set, the first pass also writes what it reads to dst.
template <int BITS, int TM, bool SPLIT, int NI, bool STAGE>
__device__ __forceinline__ void item_gateup_wide_passes(const DecodeArgs& A, const Slot& d, int i0,
                                                        const uint8_t* blob, uint8_t* dst) {
  for (int tg = 0; tg < d.ne;) {
    const int nt = min(d.ne - tg, TM);
    if (nt >= 3) gateup_pass_wide<BITS, (TM >= 3 ? 3 : 1), SPLIT, NI, STAGE>(A, d, blob, i0, tg, dst);
    else if (nt == 2) gateup_pass_wide<BITS, (TM >= 2 ? 2 : 1), SPLIT, NI, STAGE>(A, d, blob, i0, tg, dst);
    else gateup_pass_wide<BITS, 1, SPLIT, NI, STAGE>(A, d, blob, i0, tg, dst);
    tg += nt;
    dst = nullptr;
  }
}

template <int BITS, int TM, bool SPLIT, int NI, bool STAGE = false>
__device__ __forceinline__ void item_gateup_wide(const DecodeArgs& A, const Slot& d, int j,
                                                 const StageArgs* G = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i0 = (j * 4 + wave) * NI;
  if (i0 >= A.I) return;
  const int idx = resident_index(A, d.e);
  if (idx < 0) {  // expert not resident: poison its h rows
    if (lane < NI && i0 + lane < A.I)
      for (int t = 0; t < d.ne; ++t) {
        const size_t o = (size_t)(d.p0 + t) * A.I + i0 + lane;
        A.hh[o] = 0x7FC0;  // bf16 quiet NaN
        A.hl[o] = 0;
      }
    return;
  }
  const uint8_t* blob = A.base + (int64_t)idx * A.stride;
  uint8_t* dst = nullptr;
  if constexpr (STAGE) {
    // a miss: every pass reads the master copy, the first one also fills the slot
    if (const uint8_t* src = staged_source(*G, A.stride, idx)) {
      dst = const_cast<uint8_t*>(blob);
      blob = src;
    }
  }
  item_gateup_wide_passes<BITS, TM, SPLIT, NI, STAGE>(A, d, i0, blob, dst);
}

constexpr int kStageUnroll = 4;
constexpr int64_t kStageChunk = (int64_t)256 * 16 * kStageUnroll;  // bytes per copy work item

// Copy workgroup `cw` of G.ncw: work items of kStageChunk bytes over the
// missed blobs, 16 bytes per thread per step, skipping what the items write
// (those ranges start on 256-byte boundaries and their lengths are multiples
// of 128 bytes, so no 16-byte piece straddles one).
__device__ __forceinline__ void stage_copy(const StageArgs& G, uint8_t* slots, int64_t eb, int cw) {
  const int nc = *G.ncopies;
  const int64_t cpb = (eb + kStageChunk - 1) / kStageChunk;
  const int64_t total = (int64_t)nc * cpb;
  for (int64_t w = cw; w < total; w += G.ncw) {
    const int c = (int)(w / cpb);
    const int64_t ch = w % cpb;
    const uint8_t* src = G.host + (int64_t)G.copies[2 * c + 1] * eb;
    uint8_t* dst = slots + (int64_t)G.copies[2 * c] * eb;
    uint4 v[kStageUnroll];
    bool on[kStageUnroll];
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int64_t off = ch * kStageChunk + ((int64_t)u * 256 + threadIdx.x) * 16;
      bool mine = off < eb;
#pragma unroll
      for (int p = 0; p < 4; ++p) mine = mine && !(off >= G.item_lo[p] && off < G.item_hi[p]);
      on[u] = mine;
      if (mine) v[u] = *reinterpret_cast<const uint4*>(src + off);
    }
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int64_t off = ch * kStageChunk + ((int64_t)u * 256 + threadIdx.x) * 16;
      if (on[u]) *reinterpret_cast<uint4*>(dst + off) = v[u];
    }
  }
}

// stage_copy with the misses from the record of a resolve published in the
// same launch (miss_slot, miss_idx: its miss list, read into LDS).
__device__ __forceinline__ void stage_copy_list(const StageArgs& G, int nc, const int* miss_slot, const int* miss_idx,
                                                uint8_t* slots, int64_t eb, int cw) {
  const int64_t cpb = (eb + kStageChunk - 1) / kStageChunk;
  const int64_t total = (int64_t)nc * cpb;
  for (int64_t w = cw; w < total; w += G.ncw) {
    const int c = (int)(w / cpb);
    const int64_t ch = w % cpb;
    const uint8_t* src = G.host + (int64_t)miss_idx[c] * eb;
    uint8_t* dst = slots + (int64_t)miss_slot[c] * eb;
    uint4 v[kStageUnroll];
    bool on[kStageUnroll];
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int64_t off = ch * kStageChunk + ((int64_t)u * 256 + threadIdx.x) * 16;
      bool mine = off < eb;
#pragma unroll
      for (int p = 0; p < 4; ++p) mine = mine && !(off >= G.item_lo[p] && off < G.item_hi[p]);
      on[u] = mine;
      if (mine) v[u] = *reinterpret_cast<const uint4*>(src + off);
    }
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int64_t off = ch * kStageChunk + ((int64_t)u * 256 + threadIdx.x) * 16;
      if (on[u]) *reinterpret_cast<uint4*>(dst + off) = v[u];
    }
  }
}

// ---- row-tiled down with the combine folded in ------------------------------------
// One workgroup of kRowWaves waves owns kRowTile (8) output rows of H.  A wave
// takes four routed rows (sorted positions, one expert and one assignment
// each) at a time, 16 lanes per position: each lane reads its 32-column chunk
// of the position's h row once and the same chunk of the tile's rows of the
// position's down matrix, and the 16 lanes of a position then reduce the row
// sums together (a lane reading h for one position only, where lanes taking
// different rows of one position read the same h chunk four times over).  The
// y values of the tile go to global memory and to LDS, and the workgroup then
// forms out[t] = residual[t] + sum_j w[t,j] y[t,j] for its rows with the same
// fused multiply-add chain as the combine kernel.  No workgroup depends on
// another.
#ifndef MOE_ROW_TILE
#define MOE_ROW_TILE 8
#endif
constexpr int kRowTile = MOE_ROW_TILE;  // 8 or 16: one row sum per 2 or 1 of a position's 16 lanes
static_assert(kRowTile == 8 || kRowTile == 16, "rows per down workgroup");
#ifndef MOE_ROW_WAVES
#define MOE_ROW_WAVES 8
#endif
constexpr int kRowWaves = MOE_ROW_WAVES;
constexpr int kRowThreads = 64 * kRowWaves;
constexpr int kDecodeMaxRows = kDescT * kMaxK;  // routed rows a folded combine can hold (192)

// The positions pbase .. pbase + 3 (lane group qq = lane / 16 takes pbase +
// qq) over the tile's rows n0 .. n0 + kRowTile - 1.  Positions below T*k are read
// unconditionally (so that no load waits for the routed-row count; the last
// one stands in for positions past T*k); nr, the routed-row count, is
// compared only where results are stored.  The expert id read for a position
// past the routed rows is stale workspace, clamped into [0, E) so every load
// stays inside the layer.  Each row's sum goes through the same operations as
// in any other split of the rows over lanes (the same 16 chunk partials, the
// same pairing of lanes at each reduction level).
template <int BITS, bool YBF16>
__device__ __forceinline__ void down_rows_pass(const DecodeArgs& A, int pbase, int nmax, int nr, int n0,
                                               float* ylds) {
  const int lane = threadIdx.x & 63, qq = lane >> 4, gl = lane & 15;
  const int64_t rcb = (int64_t)A.I * BITS / 8, rsb = (int64_t)(A.I / 32) * 4;
  const int pq = pbase + qq;
  const int64_t pr = min(pq, nmax - 1);
  const int2 ra = *reinterpret_cast<const int2*>(A.rows + 2 * pr);  // (expert, assignment)
  const int e = min(max(ra.x, 0), A.E - 1);
  const int aa = ra.y;
  const int idx = A.pos_slot ? A.pos_slot[pr] : resident_index(A, e);
  const bool res = idx >= 0;
  const uint8_t* blob = A.base + (int64_t)(res ? idx : 0) * A.stride;
  int64_t nrow[kRowTile];
#pragma unroll
  for (int r = 0; r < kRowTile; ++r) nrow[r] = min(n0 + r, A.H - 1);
  float part[kRowTile];
#pragma unroll
  for (int r = 0; r < kRowTile; ++r) part[r] = 0.f;
  const int cpl = A.I / 512;
  for (int cc = 0; cc < cpl; ++cc) {
    const int chunk = gl + 16 * cc;
    XChunk<true> hc;
    {
      const size_t o = (size_t)pr * A.I + 32 * chunk;
      const uint4* qh = reinterpret_cast<const uint4*>(A.hh + o);
      const uint4* ql = reinterpret_cast<const uint4*>(A.hl + o);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 u = qh[i], v = ql[i];
        hc.hi[4 * i + 0] = u.x;
        hc.hi[4 * i + 1] = u.y;
        hc.hi[4 * i + 2] = u.z;
        hc.hi[4 * i + 3] = u.w;
        hc.lo[4 * i + 0] = v.x;
        hc.lo[4 * i + 1] = v.y;
        hc.lo[4 * i + 2] = v.z;
        hc.lo[4 * i + 3] = v.w;
      }
    }
    uint32_t code[kRowTile][BITS], smw[kRowTile];
#pragma unroll
    for (int r = 0; r < kRowTile; ++r) {
      load_codes<BITS, true>(code[r], blob + A.off_dc + nrow[r] * rcb + chunk * (4 * BITS));
      smw[r] = load_sm(blob + A.off_ds + nrow[r] * rsb + chunk * 4);
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sum = dot2(hc.hi[i], 0x3F803F80u, sum);
      sum = dot2(hc.lo[i], 0x3F803F80u, sum);
    }
    hc.sum = sum;
#pragma unroll
    for (int r = 0; r < kRowTile; ++r) {
      const float sc = f16lo(smw[r]), mn = f16hi(smw[r]);
      const float mo = mn - 128.0f * sc;
      part[r] = __builtin_fmaf(sc, chunk_dot<BITS, true>(code[r], hc), __builtin_fmaf(mo, sum, part[r]));
    }
  }
  // lanes of a position's 16 end with the sum of row gl * kRowTile / 16
  reduce_scatter<kRowTile, 1, 3, 0>(part, lane);
  constexpr int kLanesPerRow = 16 / kRowTile;
  if (gl % kLanesPerRow == 0 && pq < nr) {
    const int r = gl / kLanesPerRow, n = n0 + r;
    if (n < A.H) {
      const float val = res ? part[0] : __builtin_nanf("");
      float yv = val;
      if constexpr (YBF16) {
        const uint16_t b = __builtin_bit_cast(uint16_t, (__bf16)val);
        reinterpret_cast<uint16_t*>(A.y)[(int64_t)aa * A.H + n] = b;
        yv = __uint_as_float((uint32_t)b << 16);
      } else {
        reinterpret_cast<float*>(A.y)[(int64_t)aa * A.H + n] = val;
      }
      if (ylds) ylds[aa * kRowTile + r] = yv;
    }
  }
}

template <int BITS, bool YBF16>
__device__ __forceinline__ void ffn_down_rows_body(const DecodeArgs& A) {
  __shared__ float ylds[kDecodeMaxRows * kRowTile];
  __shared__ float wl[kDecodeMaxRows];
  warm_kernargs<sizeof(DecodeArgs)>();
  const int wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * kRowTile;
  const bool fold = A.out != nullptr;
  // The combine's inputs are loaded first but used only after the routed
  // rows, so no wait for them stands before the rows' loads.
  const int ct = threadIdx.x / kRowTile, cr = threadIdx.x % kRowTile;
  const bool comb = fold && ct < A.T && n0 + cr < A.H;
  const bool wmine = fold && (int)threadIdx.x < A.T * A.k;
  float wv = 0.f;
  if (wmine) wv = A.w[threadIdx.x];
  uint32_t rraw = 0;  // residual: fp32 bits, or bf16 bits in the low half
  if (comb && A.residual) {
    const size_t o = (size_t)ct * A.H + n0 + cr;
    if (A.r_bf16) rraw = reinterpret_cast<const uint16_t*>(A.residual)[o];
    else rraw = reinterpret_cast<const uint32_t*>(A.residual)[o];
  }
  // Routed rows: nr <= T*k (fewer only when dispatch dropped ids).  The loop
  // runs over T*k positions so that the row loads do not wait for nr, which
  // is read with a vector load (a scalar load's wait would come before them).
  const int nr = __builtin_nontemporal_load(A.nrows), nmax = A.T * A.k;
  float* yl = fold ? ylds : nullptr;
  for (int pbase = 4 * wave; pbase < nmax; pbase += 4 * kRowWaves) down_rows_pass<BITS, YBF16>(A, pbase, nmax, nr, n0, yl);
  if (!fold) return;
  if (wmine) wl[threadIdx.x] = wv;
  __syncthreads();
  if (comb) {
    float acc = 0.f;
    if (A.residual) acc = A.r_bf16 ? __uint_as_float(rraw << 16) : __uint_as_float(rraw);
    for (int j = 0; j < A.k; ++j) acc = __builtin_fmaf(wl[ct * A.k + j], ylds[(ct * A.k + j) * kRowTile + cr], acc);
    const size_t o = (size_t)ct * A.H + n0 + cr;
    A.out[o] = acc;
    if (A.out_bf16) {
      uint32_t u = __float_as_uint(acc);
      u += 0x7FFFu + ((u >> 16) & 1u);
      A.out_bf16[o] = (uint16_t)(u >> 16);
    }
  }
}

template <int BITS, bool YBF16>
__global__ __launch_bounds__(kRowThreads) void ffn_down_rows_kernel(DecodeArgs A) {
  ffn_down_rows_body<BITS, YBF16>(A);
}

// ---- kernels ----------------------------------------------------------------------
// Gate/up + SwiGLU: one workgroup per (active expert, tile of I).
template <int BITS, int TM, bool SPLIT, bool WIDE>
__global__ __launch_bounds__(256) void ffn_gateup_kernel(DecodeArgs A) {
  const int s = blockIdx.x / A.TA, j = blockIdx.x % A.TA;
  Slot d = load_slot(A, s);
  if (d.e < 0) return;  // slot past the active experts
  if constexpr (WIDE) {
    const int lane = threadIdx.x & 63;
    d.tokv = lane < kDescT ? d.p->tok[lane] : 0;
    item_gateup_wide<BITS, TM, SPLIT, kWideNI<SPLIT>>(A, d, j);
  }
  else item_gateup<BITS, TM, SPLIT, SPLIT ? kRLGateUpSplit<TM> : kRLGateUp<TM>>(A, d, j);
}

// Gate/up of moe_layer_decode_slots with the misses staged in the same
// launch: workgroups [0, ncw) copy, the rest are the wide gate/up items.
template <int BITS, int TM, bool SPLIT>
__global__ __launch_bounds__(256) void ffn_gateup_stage_kernel(DecodeArgs A, StageArgs G) {
  if ((int)blockIdx.x < G.ncw) {
    stage_copy(G, const_cast<uint8_t*>(A.base), A.stride, (int)blockIdx.x);
    return;
  }
  const int b = (int)blockIdx.x - G.ncw;
  const int s = b / A.TA, j = b % A.TA;
  Slot d = load_slot(A, s);
  if (d.e < 0) return;  // slot past the active experts
  const int lane = threadIdx.x & 63;
  d.tokv = lane < kDescT ? d.p->tok[lane] : 0;
  item_gateup_wide<BITS, TM, SPLIT, kWideNI<SPLIT>, true>(A, d, j, &G);
}

// Down (general shapes): one workgroup per (active expert, tile of H).
template <int BITS, int TM, bool YBF16>
__global__ __launch_bounds__(256) void ffn_down_kernel(DecodeArgs A) {
  const int s = blockIdx.x / A.TB, j = blockIdx.x % A.TB;
  const Slot d = load_slot(A, s);
  if (d.e < 0) return;  // slot past the active experts
  item_down<BITS, TM, kRLDown<TM>, YBF16>(A, d, j);
}

// Descriptors from the dispatch arrays (e = -1 for slots past n_active).
__global__ __launch_bounds__(256) void decode_prep_kernel(const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted_assign,
                                                          const int32_t* __restrict__ active,
                                                          const int32_t* __restrict__ n_active, int k, int max_active,
                                                          SlotDesc* __restrict__ desc, int32_t* __restrict__ rows,
                                                          int32_t* __restrict__ nrows) {
  const int na = *n_active;
  if (threadIdx.x == 0) *nrows = na > 0 ? offsets[active[na - 1] + 1] : 0;
  for (int s = threadIdx.x; s < max_active; s += 256) {
    SlotDesc d;
    d.e = s < na ? active[s] : -1;
    d.p0 = s < na ? offsets[d.e] : 0;
    d.ne = s < na ? offsets[d.e + 1] - d.p0 : 0;
    d.pad = 0;
    for (int j = 0; j < kDescT; ++j) {
      const int a = j < d.ne ? sorted_assign[d.p0 + j] : 0;
      d.asg[j] = a;
      d.tok[j] = a / k;
    }
    for (int j = 0; j < 4; ++j) d.pad2[j] = 0;
    desc[s] = d;
    for (int j = 0; j < d.ne; ++j) {
      rows[2 * (d.p0 + j)] = d.e;
      rows[2 * (d.p0 + j) + 1] = sorted_assign[d.p0 + j];
    }
  }
}

// The wide kernels apply when gate/up rows split over 64 lanes and down rows
// over 16 lanes in whole 32-column chunks.  Within one entry point one compiled
// pass routine (passes of up to kWideTM rows) serves every T, so a token's row
// does not depend on which other tokens share its step.  Separately compiled
// copies of a pass rounded differently while the compiler chose the fused
// multiply-adds; with contraction off and every FMA written out, the per-row
// arithmetic is the same in every instantiation, which is what lets the 2-bit
// steps of 4 to 6 tokens take a kernel with four I rows per wave (tested bit
// for bit against the four-call step at T = 4, 5 and 6).
bool wide_shape(int H, int I) { return H % 2048 == 0 && I % 512 == 0; }

template <int BITS, bool SPLIT, bool YBF16>
moe_status launch_wide(DecodeArgs& a, int max_active, hipStream_t s) {
  a.TA = (int)ceil_div(a.I, 4 * kWideNI<SPLIT>);
  launch_k(MOE_KERNEL_GEMV_GATEUP, ffn_gateup_kernel<BITS, kWideTM, SPLIT, true>,
           dim3((unsigned)(max_active * a.TA)), dim3(256), 0, s, a);
  if (moe_status st = check_launch("ffn_gateup")) return st;
  launch_k(MOE_KERNEL_GEMV_DOWN, ffn_down_rows_kernel<BITS, YBF16>, dim3((unsigned)ceil_div(a.H, kRowTile)),
           dim3(kRowThreads), 0, s, a);
  return check_launch("ffn_down");
}

// Copy workgroups of the staging gate/up launch.
constexpr int kStageCopyGroups = 64;

template <int BITS, bool SPLIT, bool YBF16>
moe_status launch_wide_stage(DecodeArgs& a, const StageArgs& g, int max_active, hipStream_t s) {
  a.TA = (int)ceil_div(a.I, 4 * kWideNI<SPLIT>);
  launch_k(MOE_KERNEL_GEMV_GATEUP, ffn_gateup_stage_kernel<BITS, kWideTM, SPLIT>,
           dim3((unsigned)(g.ncw + max_active * a.TA)), dim3(256), 0, s, a, g);
  if (moe_status st = check_launch("ffn_gateup_stage")) return st;
  launch_k(MOE_KERNEL_GEMV_DOWN, ffn_down_rows_kernel<BITS, YBF16>, dim3((unsigned)ceil_div(a.H, kRowTile)),
           dim3(kRowThreads), 0, s, a);
  return check_launch("ffn_down");
}

template <bool SPLIT, bool YBF16>
moe_status launch_stage_b(DecodeArgs& a, const StageArgs& g, int bits, int max_active, hipStream_t s) {
  return bits == 2   ? launch_wide_stage<2, SPLIT, YBF16>(a, g, max_active, s)
         : bits == 3 ? launch_wide_stage<3, SPLIT, YBF16>(a, g, max_active, s)
                     : launch_wide_stage<4, SPLIT, YBF16>(a, g, max_active, s);
}

// ---- decode step with the routing inside the gate/up launch ----------------------
// Every workgroup of the gate/up grid routes the T tokens itself (the same
// device routine as the stand-alone router, so the same bits), finds its
// active expert in LDS and goes on with its gate/up rows; workgroup 0 also
// writes the routing and dispatch outputs, which the down kernel reads after
// the launch boundary.  This replaces a launch and a descriptor load with a
// read of T*E logits that every workgroup shares through the L2.
struct RouteOut {
  const float* logits;
  int32_t *ids, *offsets, *sorted_assign, *assign_pos, *active, *n_active, *rows, *nrows;
  float* w;
};

// I rows per wave of the routed gate/up kernel: twice the stand-alone kernel's,
// so the grid (and the routing done per workgroup) is half as large and every
// workgroup is resident at once.
#ifndef MOE_ROUTED_NI
#define MOE_ROUTED_NI 8
#endif
#ifndef MOE_ROUTED_NI_SPLIT
#define MOE_ROUTED_NI_SPLIT 4
#endif
#ifndef MOE_ROUTED_NI4
#define MOE_ROUTED_NI4 4
#endif
template <int BITS, bool SPLIT>
constexpr int kRoutedNI = BITS >= 3 ? (SPLIT ? 2 : MOE_ROUTED_NI4) : (SPLIT ? MOE_ROUTED_NI_SPLIT : MOE_ROUTED_NI);

// Workgroup 0 writes the routing and dispatch outputs (the down kernel and the
// caller read them after the launch); every other workgroup routes in LDS,
// reads its slot per wave and runs its gate/up rows.
template <int BITS, bool SPLIT, int EPL, int NI>
__global__ __launch_bounds__(256) void ffn_route_gateup_kernel(DecodeArgs A, RouteOut R) {
  __shared__ dev::RouterLds L;
  warm_kernargs<sizeof(DecodeArgs) + sizeof(RouteOut)>();
  if (blockIdx.x == 0) {
    dev::decode_route_lds<EPL, 256>(R.logits, A.T, A.E, A.k, L);
    dev::decode_route_write<256>(L, A.T, A.E, A.k, R.ids, R.w, R.offsets, R.sorted_assign, R.assign_pos, R.active,
                                 R.n_active, nullptr, 0, R.rows, R.nrows);
    return;
  }
  dev::route_ids_lds<EPL, 256>(R.logits, A.T, A.E, A.k, L);
  const int b = blockIdx.x - 1, s = b / A.TA, j = b % A.TA;
  const dev::WaveSlot ws = dev::wave_slot(L, s, A.k);
  if (ws.e < 0) return;  // slot past the active experts
  item_gateup_wide<BITS, kWideTM, SPLIT, NI>(A, Slot{nullptr, ws.e, ws.p0, ws.ne, ws.tokv}, j);
}

template <int BITS, bool SPLIT, bool YBF16, int EPL, int NI = kRoutedNI<BITS, SPLIT>>
moe_status launch_wide_routed(DecodeArgs& a, const RouteOut& r, int max_active, hipStream_t s) {
  a.TA = (int)ceil_div(a.I, 4 * NI);
  launch_k(MOE_KERNEL_GEMV_GATEUP, ffn_route_gateup_kernel<BITS, SPLIT, EPL, NI>,
           dim3((unsigned)(1 + max_active * a.TA)), dim3(256), 0, s, a, r);
  if (moe_status st = check_launch("ffn_route_gateup")) return st;
  launch_k(MOE_KERNEL_GEMV_DOWN, ffn_down_rows_kernel<BITS, YBF16>, dim3((unsigned)ceil_div(a.H, kRowTile)),
           dim3(kRowThreads), 0, s, a);
  return check_launch("ffn_down");
}

// Four to six tokens (a verify step with three to five drafts) run 2-bit bf16
// steps with four I rows per wave: twice the workgroups, half the rows each,
// so the passes over an expert's tokens take half as long.  The rows' bits do
// not depend on the rows per wave.
#ifndef MOE_ROUTED_MID_T
#define MOE_ROUTED_MID_T 1
#endif
template <bool SPLIT, bool YBF16, int EPL>
moe_status launch_routed_b(DecodeArgs& a, const RouteOut& r, int bits, int max_active, hipStream_t s) {
  if (MOE_ROUTED_MID_T && bits == 2 && !SPLIT && a.T >= 4 && a.T <= 6)
    return launch_wide_routed<2, SPLIT, YBF16, EPL, 4>(a, r, max_active, s);
  return bits == 2   ? launch_wide_routed<2, SPLIT, YBF16, EPL>(a, r, max_active, s)
         : bits == 3 ? launch_wide_routed<3, SPLIT, YBF16, EPL>(a, r, max_active, s)
                     : launch_wide_routed<4, SPLIT, YBF16, EPL>(a, r, max_active, s);
}

// ---- decode step through a slot table, routing and resolve inside gate/up --------------
// moe_layer_decode_slots for the wide shapes.  Workgroup 0 routes the T
// tokens, resolves the active experts of `layer` against the table
// (dev::slot_resolve_publish: stamps and owners written, the outcome recorded,
// the table's ready word set), then writes the routing and dispatch outputs
// and the slot of each sorted position for the down launch.  Workgroups
// 1 .. ncw wait for the record and copy the parts of each missed blob that no
// gate/up item writes.  The others route the tokens themselves and run one
// gate/up item each: an expert found in the map runs from its slot at once; a
// missed one waits for the record, reads its rows from the master copy and
// writes them into its new slot as it goes.  The map, clock, miss list and
// counters are written by the down launch that follows (the map is what the
// items of this launch look experts up in).
template <int BITS, bool SPLIT, int EPL, int NI>
__global__ __launch_bounds__(256) void ffn_route_resolve_gateup_kernel(DecodeArgs A, RouteOut R, StageArgs G,
                                                                       SlotDevArgs SA, int layer, int32_t* pos_slot,
                                                                       int32_t* record) {
  __shared__ dev::RouterLds L;
  __shared__ dev::ResolveLds<256> S;
  __shared__ int published;
  const int tid = threadIdx.x, lane = tid & 63;
  dev::ResolvePrefetch<256> P;
  if (blockIdx.x == 0) {
    dev::slot_prefetch_map<256>(SA, layer, P);
    dev::slot_prefetch_stamps<256>(SA, P);
    dev::decode_route_lds<EPL, 256>(R.logits, A.T, A.E, A.k, L);
    const int na = L.na;
    dev::slot_resolve_publish<256>(SA, layer, L.slot_e, na, record, P, S);
    dev::decode_route_write<256>(L, A.T, A.E, A.k, R.ids, R.w, R.offsets, R.sorted_assign, R.assign_pos, R.active,
                                 R.n_active, nullptr, 0, R.rows, R.nrows);
    for (int s = tid; s < na; s += 256)
      for (int p = L.slot_p0[s]; p < L.slot_p0[s] + L.slot_ne[s]; ++p) pos_slot[p] = S.slot[s];
    return;
  }
  const int64_t clock = *SA.clock;  // written only between launches
  const int b = (int)blockIdx.x - 1;
  if (b < G.ncw) {
    if (!dev::slot_wait_published(SA, clock, &published)) return;
    const int nm = dev::rec_word(record, 2);
    for (int c = tid; c < nm; c += 256) {  // the miss list, in the resolve's LDS (unused here)
      S.slot[c] = dev::rec_word(record, dev::kRecMissSlot + c);
      S.rank[c] = dev::rec_word(record, dev::kRecMissIdx + c);
    }
    __syncthreads();
    stage_copy_list(G, nm, S.slot, S.rank, const_cast<uint8_t*>(A.base), A.stride, b);
    return;
  }
  dev::slot_prefetch_map<256>(SA, layer, P);
  dev::route_ids_lds<EPL, 256>(R.logits, A.T, A.E, A.k, L);
  dev::slot_map_to_lds<256>(P, S.mapl);
  __syncthreads();
  const int i = b - G.ncw, s = i / A.TA, j = i % A.TA;
  const dev::WaveSlot ws = dev::wave_slot(L, s, A.k);
  if (ws.e < 0) return;  // the same in every wave: past the active experts
  const int64_t idx = (int64_t)layer * A.E + ws.e;
  int slot = __builtin_amdgcn_readfirstlane(S.mapl[ws.e]);
  const uint8_t* master = nullptr;
  bool ok = true;
  if (slot < 0) {  // a miss: its slot comes with the record
    ok = dev::slot_wait_published(SA, clock, &published);
    if (ok) slot = __builtin_amdgcn_readfirstlane(dev::rec_word(record, dev::kRecSlot + s));
    master = G.host + idx * A.stride;
  }
  const int wave = tid >> 6, i0 = (j * 4 + wave) * NI;
  if (i0 >= A.I) return;
  if (!ok) {  // no record in time: mark this item's h rows invalid (bf16 quiet NaN)
    if (lane < NI && i0 + lane < A.I)
      for (int t = 0; t < ws.ne; ++t) {
        const size_t o = (size_t)(ws.p0 + t) * A.I + i0 + lane;
        A.hh[o] = 0x7FC0;
        A.hl[o] = 0;
      }
    return;
  }
  uint8_t* slot_blob = const_cast<uint8_t*>(A.base) + (int64_t)slot * A.stride;
  const Slot d{nullptr, ws.e, ws.p0, ws.ne, ws.tokv};
  if (!master) {
    item_gateup_wide_passes<BITS, kWideTM, SPLIT, NI, false>(A, d, i0, slot_blob, nullptr);
  } else {  // a miss: every pass reads the master copy, the first one also fills the slot (NI/2 rows at a time)
    constexpr int NH = NI > 2 ? NI / 2 : NI;
    for (int i1 = i0; i1 < i0 + NI && i1 < A.I; i1 += NH)
      item_gateup_wide_passes<BITS, kWideTM, SPLIT, NH, true>(A, d, i1, master, slot_blob);
  }
}

// Down rows of a decode step through a slot table: the slot of each sorted
// position comes from the gate/up launch (A.pos_slot); workgroup 0 also writes
// the resolve's outcome into the table state (nothing reads the old state any
// more).
template <int BITS, bool YBF16>
__global__ __launch_bounds__(kRowThreads) void ffn_down_rows_commit_kernel(DecodeArgs A, SlotDevArgs SA,
                                                                    const int32_t* record) {
  if (blockIdx.x == 0 && threadIdx.x == 0) dev::slot_record_commit(SA, record);
  ffn_down_rows_body<BITS, YBF16>(A);
}

template <int BITS, bool SPLIT, bool YBF16, int EPL, int NI = kRoutedNI<BITS, SPLIT>>
moe_status launch_resolve_routed(DecodeArgs& a, const RouteOut& r, const StageArgs& g, const SlotDevArgs& sa,
                                 int layer, int32_t* pos_slot, int32_t* record, int max_active, hipStream_t s) {
  a.TA = (int)ceil_div(a.I, 4 * NI);
  launch_k(MOE_KERNEL_GEMV_GATEUP, ffn_route_resolve_gateup_kernel<BITS, SPLIT, EPL, NI>,
           dim3((unsigned)(1 + g.ncw + max_active * a.TA)), dim3(256), 0, s, a, r, g, sa, layer, pos_slot, record);
  if (moe_status st = check_launch("ffn_route_resolve_gateup")) return st;
  a.pos_slot = pos_slot;
  launch_k(MOE_KERNEL_GEMV_DOWN, ffn_down_rows_commit_kernel<BITS, YBF16>, dim3((unsigned)ceil_div(a.H, kRowTile)),
           dim3(kRowThreads), 0, s, a, sa, (const int32_t*)record);
  return check_launch("ffn_down");
}

template <bool SPLIT, bool YBF16, int EPL>
moe_status launch_resolve_routed_b(DecodeArgs& a, const RouteOut& r, const StageArgs& g, const SlotDevArgs& sa,
                                   int layer, int32_t* pos_slot, int32_t* record, int bits, int max_active,
                                   hipStream_t s) {
  return bits == 2   ? launch_resolve_routed<2, SPLIT, YBF16, EPL>(a, r, g, sa, layer, pos_slot, record, max_active, s)
         : bits == 3 ? launch_resolve_routed<3, SPLIT, YBF16, EPL>(a, r, g, sa, layer, pos_slot, record, max_active, s)
                     : launch_resolve_routed<4, SPLIT, YBF16, EPL>(a, r, g, sa, layer, pos_slot, record, max_active, s);
}

template <int BITS, int TM, bool SPLIT, bool YBF16>
moe_status launch_tm(DecodeArgs& a, int max_active, hipStream_t s) {
  constexpr int RLA = SPLIT ? kRLGateUpSplit<TM> : kRLGateUp<TM>;
  constexpr int RLB = kRLDown<TM>;
  a.TA = (int)ceil_div(a.I, 4 * (RLA * (64 / a.ga.G) / 2));
  a.TB = (int)ceil_div(a.H, 4 * RLB * (64 / a.gb.G));
  launch_k(MOE_KERNEL_GEMV_GATEUP, ffn_gateup_kernel<BITS, TM, SPLIT, false>, dim3((unsigned)(max_active * a.TA)),
           dim3(256), 0, s, a);
  if (moe_status st = check_launch("ffn_gateup")) return st;
  launch_k(MOE_KERNEL_GEMV_DOWN, ffn_down_kernel<BITS, TM, YBF16>, dim3((unsigned)(max_active * a.TB)),
           dim3(256), 0, s, a);
  return check_launch("ffn_down");
}

template <int BITS, bool SPLIT, bool YBF16>
moe_status launch_t(DecodeArgs& a, int T, int max_active, hipStream_t s) {
  if (wide_shape(a.H, a.I)) return launch_wide<BITS, SPLIT, YBF16>(a, max_active, s);
  if (T <= 1) return launch_tm<BITS, 1, SPLIT, YBF16>(a, max_active, s);
  if (T <= 2) return launch_tm<BITS, 2, SPLIT, YBF16>(a, max_active, s);
  if (T <= 3) return launch_tm<BITS, 3, SPLIT, YBF16>(a, max_active, s);
  return launch_tm<BITS, 4, SPLIT, YBF16>(a, max_active, s);
}

template <bool SPLIT, bool YBF16>
moe_status launch_b(DecodeArgs& a, int bits, int T, int max_active, hipStream_t s) {
  return bits == 2   ? launch_t<2, SPLIT, YBF16>(a, T, max_active, s)
         : bits == 3 ? launch_t<3, SPLIT, YBF16>(a, T, max_active, s)
                     : launch_t<4, SPLIT, YBF16>(a, T, max_active, s);
}

DecodeArgs make_args(const moe_qlayer& q, const void* x, int T, int k, const int32_t* sorted_assign,
                     const int32_t* n_active, const DecodeWs& W, void* y) {
  const BlobLayout L = blob_layout(q.H, q.I, q.bits);
  DecodeArgs a{};
  a.base = reinterpret_cast<const uint8_t*>(q.base);
  a.stride = q.stride;
  a.slot_map = q.slot_map;
  a.H = q.H;
  a.I = q.I;
  a.k = k;
  a.T = T;
  a.off_gc = L.gate_codes;
  a.off_gs = L.gate_sm;
  a.off_uc = L.up_codes;
  a.off_us = L.up_sm;
  a.off_dc = L.down_codes;
  a.off_ds = L.down_sm;
  a.xin = x;
  a.n_active = n_active;
  a.desc = W.desc;
  a.sorted_assign = sorted_assign;
  a.h = W.h;
  a.hh = reinterpret_cast<uint16_t*>(W.h);
  a.hl = a.hh + (size_t)T * k * q.I;
  a.y = y;
  a.rows = W.rows;
  a.nrows = W.nrows;
  a.E = q.E;
  a.ga.G = gcd_pow2_64(q.H / 32);
  a.ga.CPL = (q.H / 32) / a.ga.G;
  a.gb.G = gcd_pow2_64(q.I / 32);
  a.gb.CPL = (q.I / 32) / a.gb.G;
  return a;
}

}  // namespace

DecodeWs decode_ws(void* ws, int T, int k, int E, int H, int I) {
  (void)H;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  uint8_t* b = reinterpret_cast<uint8_t*>(ws);
  const int n = T * k, max_active = std::min(E, n);
  DecodeWs W;
  size_t off = 0;
  W.h = reinterpret_cast<float*>(b + off);  // fp32 h, or the two bf16 planes of the wide kernels
  off += up((size_t)n * I * 4);
  W.desc = reinterpret_cast<SlotDesc*>(b + off);
  off += up((size_t)max_active * sizeof(SlotDesc));
  W.rows = reinterpret_cast<int32_t*>(b + off);
  off += up((size_t)n * 2 * 4);
  W.nrows = reinterpret_cast<int32_t*>(b + off);
  off += 256;
  W.pos_slot = reinterpret_cast<int32_t*>(b + off);
  off += up((size_t)n * 4);
  W.record = reinterpret_cast<int32_t*>(b + off);
  off += up((size_t)dev::kSlotRecordWords * 4);
  W.bytes = off;
  return W;
}

size_t ffn_gemv_ws_bytes(int T, int k, int E, int H, int I) { return decode_ws(nullptr, T, k, E, H, I).bytes; }

bool gemv_folds_combine(int H, int I) { return wide_shape(H, I); }

bool gemv_stages_misses(int H, int I) { return wide_shape(H, I); }

moe_status launch_ffn_gemv_steps(const moe_qlayer& q, const void* x, moe_dtype x_t, int T, int k,
                                 const int32_t* sorted_assign, const int32_t* n_active, const DecodeWs& W, void* y,
                                 moe_dtype y_t, const FoldedCombine& fc, hipStream_t s, const MissStage* ms) {
  DecodeArgs a = make_args(q, x, T, k, sorted_assign, n_active, W, y);
  if (fc.out) {
    if (!wide_shape(q.H, q.I) || (int64_t)T * k > kDecodeMaxRows || T * kRowTile > kRowThreads)
      return fail(MOE_EUNSUPPORTED, "combine cannot be folded for this shape");
    a.w = fc.w;
    a.residual = fc.residual;
    a.r_bf16 = fc.r_t == MOE_BF16;
    a.out = fc.out;
    a.out_bf16 = fc.out_bf16;
  }
  const int max_active = (int)std::min<int64_t>(q.E, (int64_t)T * k);
  const bool split = x_t == MOE_F32, yb = y_t == MOE_BF16;
  if (ms) {
    if (!wide_shape(q.H, q.I)) return fail(MOE_EUNSUPPORTED, "misses cannot be staged in the gate/up launch");
    const BlobLayout L = blob_layout(q.H, q.I, q.bits);
    const int64_t codes = (int64_t)q.I * q.H * q.bits / 8, sm = (int64_t)q.I * (q.H / 32) * 4;
    StageArgs g{};
    g.copies = ms->copies;
    g.ncopies = ms->ncopies;
    g.host = ms->host;
    g.item_lo[0] = L.gate_codes;
    g.item_hi[0] = L.gate_codes + codes;
    g.item_lo[1] = L.gate_sm;
    g.item_hi[1] = L.gate_sm + sm;
    g.item_lo[2] = L.up_codes;
    g.item_hi[2] = L.up_codes + codes;
    g.item_lo[3] = L.up_sm;
    g.item_hi[3] = L.up_sm + sm;
    g.ncw = kStageCopyGroups;
    if (split) return yb ? launch_stage_b<true, true>(a, g, q.bits, max_active, s)
                         : launch_stage_b<true, false>(a, g, q.bits, max_active, s);
    return yb ? launch_stage_b<false, true>(a, g, q.bits, max_active, s)
              : launch_stage_b<false, false>(a, g, q.bits, max_active, s);
  }
  if (split)
    return yb ? launch_b<true, true>(a, q.bits, T, max_active, s) : launch_b<true, false>(a, q.bits, T, max_active, s);
  return yb ? launch_b<false, true>(a, q.bits, T, max_active, s) : launch_b<false, false>(a, q.bits, T, max_active, s);
}

bool decode_routes_in_gateup(int H, int I, int T, int k) {
  return wide_shape(H, I) && (int64_t)T * k <= dev::kDecodeMaxN && T * kRowTile <= kRowThreads;
}

moe_status launch_decode_routed(const moe_qlayer& q, const float* logits, const void* x, moe_dtype x_t, int T, int k,
                                int32_t* ids, float* w, int32_t* offsets, int32_t* sorted_assign,
                                int32_t* assign_pos, int32_t* active, int32_t* n_active, const DecodeWs& W, void* y,
                                moe_dtype y_t, const FoldedCombine& fc, hipStream_t s) {
  if (!decode_routes_in_gateup(q.H, q.I, T, k) || !fc.out)
    return fail(MOE_EUNSUPPORTED, "routing cannot be fused into the gate/up launch for this shape");
  DecodeArgs a = make_args(q, x, T, k, sorted_assign, n_active, W, y);
  a.w = w;
  a.residual = fc.residual;
  a.r_bf16 = fc.r_t == MOE_BF16;
  a.out = fc.out;
  a.out_bf16 = fc.out_bf16;
  RouteOut r;
  r.logits = logits;
  r.ids = ids;
  r.w = w;
  r.offsets = offsets;
  r.sorted_assign = sorted_assign;
  r.assign_pos = assign_pos;
  r.active = active;
  r.n_active = n_active;
  r.rows = W.rows;
  r.nrows = W.nrows;
  const int max_active = (int)std::min<int64_t>(q.E, (int64_t)T * k);
  const bool split = x_t == MOE_F32, yb = y_t == MOE_BF16, big = q.E > 512;
  if (split) {
    if (yb) return big ? launch_routed_b<true, true, 16>(a, r, q.bits, max_active, s)
                       : launch_routed_b<true, true, 8>(a, r, q.bits, max_active, s);
    return big ? launch_routed_b<true, false, 16>(a, r, q.bits, max_active, s)
               : launch_routed_b<true, false, 8>(a, r, q.bits, max_active, s);
  }
  if (yb) return big ? launch_routed_b<false, true, 16>(a, r, q.bits, max_active, s)
                     : launch_routed_b<false, true, 8>(a, r, q.bits, max_active, s);
  return big ? launch_routed_b<false, false, 16>(a, r, q.bits, max_active, s)
             : launch_routed_b<false, false, 8>(a, r, q.bits, max_active, s);
}

moe_status launch_decode_routed_slots(const moe_qlayer& q, const moe_slot_table* t, int layer, const float* logits,
                                      const void* x, moe_dtype x_t, int T, int k, int32_t* ids, float* w,
                                      int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, int32_t* active,
                                      int32_t* n_active, const DecodeWs& W, void* y, moe_dtype y_t,
                                      const FoldedCombine& fc, hipStream_t s) {
  if (!decode_routes_in_gateup(q.H, q.I, T, k) || !fc.out)
    return fail(MOE_EUNSUPPORTED, "routing and resolve cannot be fused into the gate/up launch for this shape");
  DecodeArgs a = make_args(q, x, T, k, sorted_assign, n_active, W, y);
  a.w = w;
  a.residual = fc.residual;
  a.r_bf16 = fc.r_t == MOE_BF16;
  a.out = fc.out;
  a.out_bf16 = fc.out_bf16;
  RouteOut r;
  r.logits = logits;
  r.ids = ids;
  r.w = w;
  r.offsets = offsets;
  r.sorted_assign = sorted_assign;
  r.assign_pos = assign_pos;
  r.active = active;
  r.n_active = n_active;
  r.rows = W.rows;
  r.nrows = W.nrows;
  const SlotTableView v = slot_table_view(t);
  const BlobLayout L = blob_layout(q.H, q.I, q.bits);
  const int64_t codes = (int64_t)q.I * q.H * q.bits / 8, sm = (int64_t)q.I * (q.H / 32) * 4;
  StageArgs g{};
  g.host = v.host_dev;
  g.item_lo[0] = L.gate_codes;
  g.item_hi[0] = L.gate_codes + codes;
  g.item_lo[1] = L.gate_sm;
  g.item_hi[1] = L.gate_sm + sm;
  g.item_lo[2] = L.up_codes;
  g.item_hi[2] = L.up_codes + codes;
  g.item_lo[3] = L.up_sm;
  g.item_hi[3] = L.up_sm + sm;
  g.ncw = kStageCopyGroups;
  const SlotDevArgs sa = slot_dev_args(t);
  const int max_active = (int)std::min<int64_t>(q.E, (int64_t)T * k);
  const bool split = x_t == MOE_F32, yb = y_t == MOE_BF16, big = q.E > 512;
  if (split) {
    if (yb) return big ? launch_resolve_routed_b<true, true, 16>(a, r, g, sa, layer, W.pos_slot, W.record, q.bits, max_active, s)
                       : launch_resolve_routed_b<true, true, 8>(a, r, g, sa, layer, W.pos_slot, W.record, q.bits, max_active, s);
    return big ? launch_resolve_routed_b<true, false, 16>(a, r, g, sa, layer, W.pos_slot, W.record, q.bits, max_active, s)
               : launch_resolve_routed_b<true, false, 8>(a, r, g, sa, layer, W.pos_slot, W.record, q.bits, max_active, s);
  }
  if (yb) return big ? launch_resolve_routed_b<false, true, 16>(a, r, g, sa, layer, W.pos_slot, W.record, q.bits, max_active, s)
                     : launch_resolve_routed_b<false, true, 8>(a, r, g, sa, layer, W.pos_slot, W.record, q.bits, max_active, s);
  return big ? launch_resolve_routed_b<false, false, 16>(a, r, g, sa, layer, W.pos_slot, W.record, q.bits, max_active, s)
             : launch_resolve_routed_b<false, false, 8>(a, r, g, sa, layer, W.pos_slot, W.record, q.bits, max_active, s);
}

moe_status launch_ffn_gemv(const moe_qlayer& q, const void* x, moe_dtype x_t, int T, int k, const int32_t* offsets,
                           const int32_t* sorted_assign, const int32_t* active, const int32_t* n_active, void* y,
                           moe_dtype y_t, void* ws, hipStream_t s) {
  const DecodeWs W = decode_ws(ws, T, k, q.E, q.H, q.I);
  const int max_active = (int)std::min<int64_t>(q.E, (int64_t)T * k);
  launch_k(MOE_KERNEL_DECODE_PREP, decode_prep_kernel, dim3(1), dim3(256), 0, s, offsets, sorted_assign, active,
           n_active, k, max_active, W.desc, W.rows, W.nrows);
  if (moe_status st = check_launch("decode_prep")) return st;
  return launch_ffn_gemv_steps(q, x, x_t, T, k, sorted_assign, n_active, W, y, y_t, FoldedCombine{}, s);
}

}  // namespace moe
