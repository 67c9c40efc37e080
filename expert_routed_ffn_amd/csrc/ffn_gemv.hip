// ffn_gemv.hip -- expert FFN for decode and verify steps (few tokens per expert).
//
// Passage: only the routed experts' weights are touched per token (Strata
// feature, tech.hub77a.com, summary row "핵심 기법" and section "2. 왜 대단한가"
// (1)); verify steps run 1 + d tokens through the model at once (same page,
// (3)); the fast size is a 2-bit class quantization (section "3. 바로 써먹기").
//
// For each active expert e and each of its n_e routed rows x:
//   g = Wg x, u = Wu x, h = silu(g) * u    (h kept in fp32)
//   y = Wd h                               (written per assignment)
// and, in the fused decode step, out[t] = residual[t] + sum_j w[t,j] y[t,j].
//
// Arithmetic per block of 32 weights (scale s, min m, codes q):
//   sum_c (s*q_c + m) x_c = s * sum_c (128 + q_c) x_c + (m - 128*s) * sum_c x_c.
// (128 + q) is a bf16 whose bit pattern is 0x4300 | q, so two codes become a
// packed bf16 pair with one shift and one and-or (the code layout puts
// adjacent columns in the two halfwords of a word), and v_dot2c_f32_bf16 does
// the two MACs against the packed input pair with fp32 accumulation.
// sum_c x_c is per input row and chunk, computed once per wave.  Inputs that
// are not bf16 (fp32 activations, the fp32 h) are carried as an unevaluated
// sum hi + lo of two bf16 values (about 16 significant bits), so the products
// stay exact and accumulation is fp32.
//
// Work split.  A row of K weights is cut into K/32 chunks (one scale/min block
// each).  G lanes share a row (G = gcd(K/32, 64)), each lane owning K/(32G)
// chunks; a wave covers 64/G rows per step and RL steps, and every lane issues
// the loads of all its RL rows before any arithmetic.  Lane partial sums are
// reduced across the G lanes with xor shuffles.  Gate row i and up row i land
// in the same lane, so SwiGLU is applied right after the reduction.
//
// Scheduling.  A decode step moves ~20 MB, a few microseconds of HBM time, so
// launch and dependency latency dominate.  Every (active expert, row tile) is
// one workgroup and all of them are resident at once; a per-expert
// descriptor (id, first row, row count, tokens) built by the preceding
// single-workgroup kernel lets a workgroup reach its weights and inputs after
// one dependent load.  In the fused decode step the combine is folded into
// the down kernel: the workgroup that completes a (token, column tile) cell
// last sums that cell's k rows into out.
#include "internal.hpp"

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

// y rows handed to the workgroup that combines them, inside one launch, are
// written and read with agent-scope relaxed atomics: plain stores and loads
// with the agent-coherence bit, so no whole-cache write-back or invalidate is
// needed.  The hand-off is: every wave waits for its stores to complete, a
// barrier, then a relaxed counter increment; the last of the k contributors
// to a cell reads the rows after a barrier.
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint16_t ld_coherent(const uint16_t* p) {
  return __hip_atomic_load(const_cast<uint16_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  constexpr uint32_t kMask = BITS == 2 ? 0x00030003u : 0x000F000Fu;
  constexpr int kPairs = 16 / BITS;  // code pairs per word
  float acc = 0.f;
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

template <int BITS>
__device__ __forceinline__ void load_codes(uint32_t (&code)[BITS], const uint8_t* p) {
  if constexpr (BITS == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    code[0] = v.x;
    code[1] = v.y;
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    code[0] = v.x;
    code[1] = v.y;
    code[2] = v.z;
    code[3] = v.w;
  }
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
  int32_t* done;
  int32_t* cnt;
  int32_t* flag;
  float* h;
  void* y;
  const float* w;
  const void* residual;
  int r_bf16;
  float* out;
  uint16_t* out_bf16;
  int TA, TB;  // gate/up and down items per expert
  Geo ga, gb;
};

// One active expert as an item sees it: scalars plus the descriptor in memory
// (its token lists are read through the pointer, never copied into an
// indexed local array).
struct Slot {
  const SlotDesc* p;
  int e, p0, ne;
};

__device__ __forceinline__ Slot load_slot(const DecodeArgs& A, int s) {
  const SlotDesc* p = A.desc + s;
  return Slot{p, p->e, p->p0, p->ne};
}

// Token and assignment of the rel-th routed row of a slot.
__device__ __forceinline__ int row_token(const DecodeArgs& A, const Slot& d, int rel) {
  return rel < kDescT ? d.p->tok[rel] : A.sorted_assign[d.p0 + rel] / A.k;
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
      load_codes<BITS>(code[r], blob + (up ? A.off_uc : A.off_gc) + i * row_code_bytes + chunk * (4 * BITS));
      smw[r] = *reinterpret_cast<const uint32_t*>(blob + (up ? A.off_us : A.off_gs) + i * row_sm_bytes + chunk * 4);
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
      for (int t = 0; t < NT; ++t) part[r][t] += s * chunk_dot<BITS, SPLIT>(code[r], xc[t]) + mo * xc[t].sum;
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

// ---- down -----------------------------------------------------------------------
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
    load_codes<BITS>(P.code[r], blob + A.off_dc + n * row_code_bytes + chunk * (4 * BITS));
    P.smw[r] = *reinterpret_cast<const uint32_t*>(blob + A.off_ds + n * row_sm_bytes + chunk * 4);
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
    for (int t = 0; t < NT; ++t) part[r][t] += s * chunk_dot<BITS, true>(P.code[r], hc[t]) + mo * hc[t].sum;
  }
}

// One pass over the wave's down rows for NT routed rows; chunk 0's weights
// come from `pre` when have_pre (issued before the wait), the rest are loaded.
template <int BITS, int NT, int RL, bool YBF16, bool COHERENT>
__device__ __forceinline__ void down_pass(const DecodeArgs& A, const Slot& d, const uint8_t* blob, int n0,
                                          int rel0, bool resident, const DownPre<BITS, RL>& pre, bool have_pre) {
  const int lane = threadIdx.x & 63;
  const int G = A.gb.G, RPI = 64 / G, sl = lane / G, gl = lane % G;
  float part[RL][NT];
#pragma unroll
  for (int r = 0; r < RL; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) part[r][t] = 0.f;

  if (resident) {
    if (have_pre) {
      down_chunk<BITS, NT, RL>(A, d, rel0, 0, pre, part);
    } else {
      DownPre<BITS, RL> P;
      down_load<BITS, RL>(A, blob, n0, 0, P);
      down_chunk<BITS, NT, RL>(A, d, rel0, 0, P, part);
    }
    for (int cc = 1; cc < A.gb.CPL; ++cc) {
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
        if constexpr (YBF16) {
          const uint16_t b = __builtin_bit_cast(uint16_t, (__bf16)v);
          if constexpr (COHERENT) st_coherent(&reinterpret_cast<uint16_t*>(A.y)[a * A.H + n], b);
          else reinterpret_cast<uint16_t*>(A.y)[a * A.H + n] = b;
        } else {
          if constexpr (COHERENT) st_coherent(&reinterpret_cast<float*>(A.y)[a * A.H + n], v);
          else reinterpret_cast<float*>(A.y)[a * A.H + n] = v;
        }
      }
    }
  }
}

// Combine one (token, column range) cell: out = residual + sum_j w_j y_j, j ascending.
template <bool YBF16>
__device__ __forceinline__ void combine_cell(const DecodeArgs& A, int t, int c0, int c1) {
  for (int c = c0 + (int)threadIdx.x; c < c1; c += 256) {
    float acc = 0.f;
    if (A.residual)
      acc = A.r_bf16
                ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(A.residual)[(size_t)t * A.H + c] << 16)
                : reinterpret_cast<const float*>(A.residual)[(size_t)t * A.H + c];
    for (int j = 0; j < A.k; ++j) {
      const float wj = A.w[(size_t)t * A.k + j];
      const size_t yi = ((size_t)t * A.k + j) * A.H + c;
      const float yv = YBF16 ? __uint_as_float((uint32_t)ld_coherent(&reinterpret_cast<const uint16_t*>(A.y)[yi]) << 16)
                             : ld_coherent(&reinterpret_cast<const float*>(A.y)[yi]);
      acc += wj * yv;
    }
    A.out[(size_t)t * A.H + c] = acc;
    if (A.out_bf16) {
      uint32_t u = __float_as_uint(acc);
      u += 0x7FFFu + ((u >> 16) & 1u);
      A.out_bf16[(size_t)t * A.H + c] = (uint16_t)(u >> 16);
    }
  }
}

template <int BITS, int TM, int RL, bool YBF16, bool COMBINE>
__device__ __forceinline__ void item_down(const DecodeArgs& A, const Slot& d, int j) {
  const int wave = threadIdx.x >> 6;
  const int RPI = 64 / A.gb.G;
  const int n0 = (j * 4 + wave) * RL * RPI;
  const int idx = resident_index(A, d.e);
  const bool resident = idx >= 0;
  const uint8_t* blob = A.base + (int64_t)(resident ? idx : 0) * A.stride;
  if (n0 < A.H) {
    DownPre<BITS, RL> none;
    for (int tg = 0; tg < d.ne;) {
      const int nt = min(d.ne - tg, TM);
      if (nt >= 4) down_pass<BITS, (TM >= 4 ? 4 : 1), RL, YBF16, COMBINE>(A, d, blob, n0, tg, resident, none, false);
      else if (nt == 3) down_pass<BITS, (TM >= 3 ? 3 : 1), RL, YBF16, COMBINE>(A, d, blob, n0, tg, resident, none, false);
      else if (nt == 2) down_pass<BITS, (TM >= 2 ? 2 : 1), RL, YBF16, COMBINE>(A, d, blob, n0, tg, resident, none, false);
      else down_pass<BITS, 1, RL, YBF16, COMBINE>(A, d, blob, n0, tg, resident, none, false);
      tg += nt;
    }
  }

  if constexpr (COMBINE) {
    __shared__ int last[kDescT];
    __builtin_amdgcn_s_waitcnt(0);  // this wave's y stores are complete
    __syncthreads();
    if ((int)threadIdx.x < d.ne) {
      const int t = d.p->tok[threadIdx.x];
      const int old = __hip_atomic_fetch_add(&A.cnt[t * A.TB + j], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last[threadIdx.x] = (old == A.k - 1) ? t : -1;
    }
    __syncthreads();
    const int c0 = j * 4 * RL * RPI, c1 = min(A.H, c0 + 4 * RL * RPI);
    for (int q = 0; q < d.ne; ++q)
      if (last[q] >= 0) combine_cell<YBF16>(A, last[q], c0, c1);
  }
}

// Gate/up + SwiGLU: one workgroup per (active expert, tile of I).
template <int BITS, int TM, bool SPLIT>
__global__ __launch_bounds__(256) void ffn_gateup_kernel(DecodeArgs A) {
  constexpr int RLA = SPLIT ? kRLGateUpSplit<TM> : kRLGateUp<TM>;
  const int s = blockIdx.x / A.TA, j = blockIdx.x % A.TA;
  if (s >= *A.n_active) return;
  const Slot d = load_slot(A, s);
  item_gateup<BITS, TM, SPLIT, RLA>(A, d, j);
}

// Down (+ combine): one workgroup per (active expert, tile of H).
template <int BITS, int TM, bool YBF16, bool COMBINE>
__global__ __launch_bounds__(256) void ffn_down_kernel(DecodeArgs A) {
  constexpr int RLB = kRLDown<TM>;
  const int s = blockIdx.x / A.TB, j = blockIdx.x % A.TB;
  if (s >= *A.n_active) return;
  const Slot d = load_slot(A, s);
  item_down<BITS, TM, RLB, YBF16, COMBINE>(A, d, j);
}

// Descriptors from the dispatch arrays, and counters cleared.
__global__ __launch_bounds__(256) void decode_prep_kernel(const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted_assign,
                                                          const int32_t* __restrict__ active,
                                                          const int32_t* __restrict__ n_active, int k, int max_active,
                                                          SlotDesc* __restrict__ desc, int32_t* __restrict__ done,
                                                          int32_t* __restrict__ cnt, int n_cnt,
                                                          int32_t* __restrict__ flag) {
  const int na = *n_active;
  for (int s = threadIdx.x; s < max_active; s += 256) {
    done[s] = 0;
    if (s >= na) continue;
    SlotDesc d;
    d.e = active[s];
    d.p0 = offsets[d.e];
    d.ne = offsets[d.e + 1] - d.p0;
    d.pad = 0;
    for (int j = 0; j < kDescT; ++j) {
      const int a = j < d.ne ? sorted_assign[d.p0 + j] : 0;
      d.asg[j] = a;
      d.tok[j] = a / k;
    }
    for (int j = 0; j < 4; ++j) d.pad2[j] = 0;
    desc[s] = d;
  }
  for (int i = threadIdx.x; i < n_cnt; i += 256) cnt[i] = 0;
  if (threadIdx.x == 0) *flag = 0;
}

template <int BITS, int TM, bool SPLIT, bool YBF16, bool COMBINE>
moe_status launch_tm(DecodeArgs& a, int max_active, hipStream_t s) {
  constexpr int RLA = SPLIT ? kRLGateUpSplit<TM> : kRLGateUp<TM>;
  constexpr int RLB = kRLDown<TM>;
  const int NI = RLA * (64 / a.ga.G) / 2;
  a.TA = (int)ceil_div(a.I, 4 * NI);
  a.TB = (int)ceil_div(a.H, 4 * RLB * (64 / a.gb.G));
  launch_k(MOE_KERNEL_GEMV_GATEUP, ffn_gateup_kernel<BITS, TM, SPLIT>, dim3((unsigned)(max_active * a.TA)), dim3(256),
           0, s, a);
  if (moe_status st = check_launch("ffn_gateup")) return st;
  launch_k(MOE_KERNEL_GEMV_DOWN, ffn_down_kernel<BITS, TM, YBF16, COMBINE>, dim3((unsigned)(max_active * a.TB)),
           dim3(256), 0, s, a);
  return check_launch("ffn_down");
}

template <int BITS, bool SPLIT, bool YBF16, bool COMBINE>
moe_status launch_t(DecodeArgs& a, int T, int max_active, hipStream_t s) {
  if (T <= 1) return launch_tm<BITS, 1, SPLIT, YBF16, COMBINE>(a, max_active, s);
  if (T <= 2) return launch_tm<BITS, 2, SPLIT, YBF16, COMBINE>(a, max_active, s);
  if (T <= 3) return launch_tm<BITS, 3, SPLIT, YBF16, COMBINE>(a, max_active, s);
  return launch_tm<BITS, 4, SPLIT, YBF16, COMBINE>(a, max_active, s);
}

template <bool SPLIT, bool YBF16, bool COMBINE>
moe_status launch_b(DecodeArgs& a, int bits, int T, int max_active, hipStream_t s) {
  return bits == 2 ? launch_t<2, SPLIT, YBF16, COMBINE>(a, T, max_active, s)
                   : launch_t<4, SPLIT, YBF16, COMBINE>(a, T, max_active, s);
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
  a.done = W.done;
  a.cnt = W.cnt;
  a.flag = W.flag;
  a.h = W.h;
  a.y = y;
  a.ga.G = gcd_pow2_64(q.H / 32);
  a.ga.CPL = (q.H / 32) / a.ga.G;
  a.gb.G = gcd_pow2_64(q.I / 32);
  a.gb.CPL = (q.I / 32) / a.gb.G;
  return a;
}

}  // namespace

DecodeWs decode_ws(void* ws, int T, int k, int E, int H, int I) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  uint8_t* b = reinterpret_cast<uint8_t*>(ws);
  const int n = T * k, max_active = std::min(E, n);
  DecodeWs W;
  size_t off = 0;
  W.h = reinterpret_cast<float*>(b + off);
  off += up((size_t)n * I * 4);
  W.desc = reinterpret_cast<SlotDesc*>(b + off);
  off += up((size_t)max_active * sizeof(SlotDesc));
  W.done = reinterpret_cast<int32_t*>(b + off);
  off += up((size_t)max_active * 4);
  W.n_cnt = T * (int)ceil_div(H, 16);
  W.cnt = reinterpret_cast<int32_t*>(b + off);
  off += up((size_t)W.n_cnt * 4);
  W.flag = reinterpret_cast<int32_t*>(b + off);
  off += 256;
  W.bytes = off;
  return W;
}

size_t ffn_gemv_ws_bytes(int T, int k, int E, int H, int I) { return decode_ws(nullptr, T, k, E, H, I).bytes; }

moe_status launch_ffn_gemv_fused(const moe_qlayer& q, const void* x, moe_dtype x_t, int T, int k,
                                 const int32_t* sorted_assign, const int32_t* n_active, const DecodeWs& W, void* y,
                                 moe_dtype y_t, const float* w, const void* residual, moe_dtype r_t, float* out,
                                 uint16_t* out_bf16, bool combine, hipStream_t s) {
  DecodeArgs a = make_args(q, x, T, k, sorted_assign, n_active, W, y);
  a.w = w;
  a.residual = residual;
  a.r_bf16 = r_t == MOE_BF16;
  a.out = out;
  a.out_bf16 = out_bf16;
  const int max_active = (int)std::min<int64_t>(q.E, (int64_t)T * k);
  const bool split = x_t == MOE_F32, yb = y_t == MOE_BF16;
  if (combine) {
    if (split)
      return yb ? launch_b<true, true, true>(a, q.bits, T, max_active, s)
                : launch_b<true, false, true>(a, q.bits, T, max_active, s);
    return yb ? launch_b<false, true, true>(a, q.bits, T, max_active, s)
              : launch_b<false, false, true>(a, q.bits, T, max_active, s);
  }
  if (split)
    return yb ? launch_b<true, true, false>(a, q.bits, T, max_active, s)
              : launch_b<true, false, false>(a, q.bits, T, max_active, s);
  return yb ? launch_b<false, true, false>(a, q.bits, T, max_active, s)
            : launch_b<false, false, false>(a, q.bits, T, max_active, s);
}

moe_status launch_ffn_gemv(const moe_qlayer& q, const void* x, moe_dtype x_t, int T, int k, const int32_t* offsets,
                           const int32_t* sorted_assign, const int32_t* active, const int32_t* n_active, void* y,
                           moe_dtype y_t, void* ws, hipStream_t s) {
  const DecodeWs W = decode_ws(ws, T, k, q.E, q.H, q.I);
  const int max_active = (int)std::min<int64_t>(q.E, (int64_t)T * k);
  launch_k(MOE_KERNEL_DECODE_PREP, decode_prep_kernel, dim3(1), dim3(256), 0, s, offsets, sorted_assign, active,
           n_active, k, max_active, W.desc, W.done, W.cnt, W.n_cnt, W.flag);
  if (moe_status st = check_launch("decode_prep")) return st;
  return launch_ffn_gemv_fused(q, x, x_t, T, k, sorted_assign, n_active, W, y, y_t, nullptr, nullptr, MOE_F32, nullptr,
                               nullptr, false, s);
}

}  // namespace moe
