// ffn_gemv.hip -- expert FFN for decode and verify steps (few tokens per expert).
//
// Passage: only the routed experts' weights are touched per token (Strata
// feature, tech.hub77a.com, summary row "핵심 기법" and section "2. 왜 대단한가"
// (1)); verify steps run 1 + d tokens through the model at once (same page,
// (3)); the fast size is a 2-bit class quantization (section "3. 바로 써먹기").
//
// For each active expert e and each of its n_e routed rows x:
//   g = Wg x, u = Wu x, h = silu(g) * u         (kernel 1, h kept in fp32)
//   y = Wd h                                    (kernel 2, y written per assignment)
// With n_e <= 8 every weight feeds only a few MACs, so the kernels are bound
// by streaming the packed weights from HBM: the work per weight must stay
// within a couple of VALU ops.
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
// the loads of all its RL rows before doing any arithmetic, so each wave keeps
// RL * 12 bytes per lane in flight.  Lane partial sums are reduced across the
// G lanes with xor shuffles.  Gate row i and up row i land in the same lane, so
// SwiGLU is applied right after the reduction.
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
// and the exact-ish chunk sum.
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

template <bool SPLIT>
__device__ __forceinline__ void zero_chunk(XChunk<SPLIT>& c) {
#pragma unroll
  for (int i = 0; i < 16; ++i) c.hi[i] = 0u;
#pragma unroll
  for (int i = 0; i < (SPLIT ? 16 : 1); ++i) c.lo[i] = 0u;
  c.sum = 0.f;
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
      const uint32_t v = ((code[d] >> (BITS * p)) & kMask) | 0x43004300u;
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

__host__ __device__ inline int gcd_pow2_64(int nc) {
  int g = 1;
  while (g < 64 && nc % (2 * g) == 0) g *= 2;
  return g;
}

// ---------------------------------------------------------------------------
// Kernel 1: h = silu(Wg x) * (Wu x) for every (expert, routed row).
// Grid: max_active * tiles.  Block: 4 waves.  A wave owns NI = RL*RPI/2
// consecutive i; lane row r (rho = r*RPI + sl) is gate row i0 + rho for
// rho < NI and up row i0 + rho - NI otherwise, so gate and up of one i meet
// in the same lane (rows r and r + RL/2).
// ---------------------------------------------------------------------------
struct GateUpArgs {
  const uint8_t* blob;
  int64_t off_gc, off_gs, off_uc, off_us;
  int H, I, k, i0, NI, RPI, sl, gl, G, CPL;
  const void* xin;
  const int32_t* sorted_assign;
  float* h_ws;
};

// One pass over the wave's rows for the NT routed rows at sorted positions p .. p+NT-1.
template <int BITS, int NT, bool SPLIT, int RL>
__device__ __forceinline__ void gateup_pass(const GateUpArgs& A, int p) {
  const int64_t row_code_bytes = (int64_t)A.H * BITS / 8, row_sm_bytes = (int64_t)(A.H / 32) * 4;
  int64_t tok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) tok[t] = A.sorted_assign[p + t] / A.k;

  float part[RL][NT];
#pragma unroll
  for (int r = 0; r < RL; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) part[r][t] = 0.f;

  for (int cc = 0; cc < A.CPL; ++cc) {
    const int chunk = A.gl + A.G * cc;
    uint32_t code[RL][BITS];
    uint32_t smw[RL];
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      const int rho = r * A.RPI + A.sl;
      const bool up = rho >= A.NI;
      int i = A.i0 + (up ? rho - A.NI : rho);
      i = i < A.I ? i : A.I - 1;  // rows past I are computed on a valid row and dropped
      load_codes<BITS>(code[r], A.blob + (up ? A.off_uc : A.off_gc) + i * row_code_bytes + chunk * (4 * BITS));
      smw[r] = *reinterpret_cast<const uint32_t*>(A.blob + (up ? A.off_us : A.off_gs) + i * row_sm_bytes + chunk * 4);
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
    for (int t = 0; t < NT; ++t) part[r][t] = group_sum(part[r][t], A.G);

  if (A.gl == 0) {
#pragma unroll
    for (int r = 0; r < RL / 2; ++r) {
      const int i = A.i0 + r * A.RPI + A.sl;
      if (i >= A.I) continue;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float g = part[r][t], u = part[r + RL / 2][t];
        A.h_ws[(size_t)(p + t) * A.I + i] = g / (1.0f + expf(-g)) * u;
      }
    }
  }
}

template <int BITS, int TM, bool SPLIT, int RL>
__global__ __launch_bounds__(256) void ffn_gateup_kernel(
    const uint8_t* __restrict__ base, int64_t stride, const int32_t* __restrict__ slot_map, int H, int I,
    int64_t off_gc, int64_t off_gs, int64_t off_uc, int64_t off_us, const void* __restrict__ xin,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_assign, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, int k, int tiles, Geo geo, float* __restrict__ h_ws) {
  const int slot = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  if (slot >= *n_active) return;
  const int e = active[slot];
  const int p0 = offsets[e], ne = offsets[e + 1] - p0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  GateUpArgs A;
  A.G = geo.G;
  A.CPL = geo.CPL;
  A.RPI = 64 / A.G;
  A.sl = lane / A.G;
  A.gl = lane % A.G;
  A.NI = RL * A.RPI / 2;
  A.i0 = (tile * 4 + wave) * A.NI;
  if (A.i0 >= I) return;
  const int idx = slot_map ? slot_map[e] : e;
  if (idx < 0) {  // expert not resident: poison its h rows
    for (int r = 0; r < RL / 2; ++r) {
      const int i = A.i0 + r * A.RPI + A.sl;
      if (A.gl == 0 && i < I)
        for (int t = 0; t < ne; ++t) h_ws[(size_t)(p0 + t) * I + i] = __builtin_nanf("");
    }
    return;
  }
  A.blob = base + (int64_t)idx * stride;
  A.off_gc = off_gc;
  A.off_gs = off_gs;
  A.off_uc = off_uc;
  A.off_us = off_us;
  A.H = H;
  A.I = I;
  A.k = k;
  A.xin = xin;
  A.sorted_assign = sorted_assign;
  A.h_ws = h_ws;
  for (int tg = 0; tg < ne;) {
    const int nt = min(ne - tg, TM);
    if (nt >= 4) gateup_pass<BITS, (TM >= 4 ? 4 : 1), SPLIT, RL>(A, p0 + tg);
    else if (nt == 3) gateup_pass<BITS, (TM >= 4 ? 3 : 1), SPLIT, RL>(A, p0 + tg);
    else if (nt == 2) gateup_pass<BITS, (TM >= 2 ? 2 : 1), SPLIT, RL>(A, p0 + tg);
    else gateup_pass<BITS, 1, SPLIT, RL>(A, p0 + tg);
    tg += nt;
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: y[a] = Wd h for every (expert, routed row).  Lane row r is output
// row n0 + r*RPI + sl.
// ---------------------------------------------------------------------------
struct DownArgs {
  const uint8_t* blob;
  int64_t off_dc, off_ds;
  int H, I, n0, RPI, sl, gl, G, CPL;
  const float* h_ws;
  const int32_t* sorted_assign;
  void* y;
};

template <int BITS, int NT, int RL, bool YBF16>
__device__ __forceinline__ void down_pass(const DownArgs& A, int p, bool resident) {
  const int64_t row_code_bytes = (int64_t)A.I * BITS / 8, row_sm_bytes = (int64_t)(A.I / 32) * 4;
  float part[RL][NT];
#pragma unroll
  for (int r = 0; r < RL; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) part[r][t] = 0.f;

  if (resident) {
    for (int cc = 0; cc < A.CPL; ++cc) {
      const int chunk = A.gl + A.G * cc;
      uint32_t code[RL][BITS];
      uint32_t smw[RL];
#pragma unroll
      for (int r = 0; r < RL; ++r) {
        int n = A.n0 + r * A.RPI + A.sl;
        n = n < A.H ? n : A.H - 1;
        load_codes<BITS>(code[r], A.blob + A.off_dc + n * row_code_bytes + chunk * (4 * BITS));
        smw[r] = *reinterpret_cast<const uint32_t*>(A.blob + A.off_ds + n * row_sm_bytes + chunk * 4);
      }
      XChunk<true> hc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) load_chunk(hc[t], A.h_ws + (size_t)(p + t) * A.I + 32 * chunk);
#pragma unroll
      for (int r = 0; r < RL; ++r) {
        const float s = f16lo(smw[r]), m = f16hi(smw[r]);
        const float mo = m - 128.0f * s;
#pragma unroll
        for (int t = 0; t < NT; ++t) part[r][t] += s * chunk_dot<BITS, true>(code[r], hc[t]) + mo * hc[t].sum;
      }
    }
  }

#pragma unroll
  for (int r = 0; r < RL; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) part[r][t] = group_sum(part[r][t], A.G);

  if (A.gl == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t a = A.sorted_assign[p + t];
#pragma unroll
      for (int r = 0; r < RL; ++r) {
        const int n = A.n0 + r * A.RPI + A.sl;
        if (n >= A.H) continue;
        const float v = resident ? part[r][t] : __builtin_nanf("");
        if constexpr (YBF16)
          reinterpret_cast<uint16_t*>(A.y)[a * A.H + n] = __builtin_bit_cast(uint16_t, (__bf16)v);
        else
          reinterpret_cast<float*>(A.y)[a * A.H + n] = v;
      }
    }
  }
}

template <int BITS, int TM, int RL, bool YBF16>
__global__ __launch_bounds__(256) void ffn_down_kernel(
    const uint8_t* __restrict__ base, int64_t stride, const int32_t* __restrict__ slot_map, int H, int I,
    int64_t off_dc, int64_t off_ds, const float* __restrict__ h_ws, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_assign, const int32_t* __restrict__ active, const int32_t* __restrict__ n_active,
    int tiles, Geo geo, void* __restrict__ yout) {
  const int slot = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  if (slot >= *n_active) return;
  const int e = active[slot];
  const int p0 = offsets[e], ne = offsets[e + 1] - p0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  DownArgs A;
  A.G = geo.G;
  A.CPL = geo.CPL;
  A.RPI = 64 / A.G;
  A.sl = lane / A.G;
  A.gl = lane % A.G;
  A.n0 = (tile * 4 + wave) * RL * A.RPI;
  if (A.n0 >= H) return;
  const int idx = slot_map ? slot_map[e] : e;
  A.blob = base + (int64_t)(idx < 0 ? 0 : idx) * stride;
  A.off_dc = off_dc;
  A.off_ds = off_ds;
  A.H = H;
  A.I = I;
  A.h_ws = h_ws;
  A.sorted_assign = sorted_assign;
  A.y = yout;
  const bool resident = idx >= 0;
  for (int tg = 0; tg < ne;) {
    const int nt = min(ne - tg, TM);
    if (nt >= 4) down_pass<BITS, (TM >= 4 ? 4 : 1), RL, YBF16>(A, p0 + tg, resident);
    else if (nt == 3) down_pass<BITS, (TM >= 4 ? 3 : 1), RL, YBF16>(A, p0 + tg, resident);
    else if (nt == 2) down_pass<BITS, (TM >= 2 ? 2 : 1), RL, YBF16>(A, p0 + tg, resident);
    else down_pass<BITS, 1, RL, YBF16>(A, p0 + tg, resident);
    tg += nt;
  }
}

// Rows per lane: as many as registers allow without dropping below two waves per SIMD.
template <int TM> constexpr int kRLGateUp = TM >= 4 ? 8 : 16;
template <int TM> constexpr int kRLGateUpSplit = TM >= 4 ? 4 : 8;
template <int TM> constexpr int kRLDown = TM >= 4 ? 4 : 8;

template <int BITS, int TM>
moe_status launch_bits_tm(const moe_qlayer& q, const BlobLayout& L, const void* x, bool split, int k,
                          const int32_t* offsets, const int32_t* sorted_assign, const int32_t* active,
                          const int32_t* n_active, int max_active, void* y, bool ybf16, float* h_ws, hipStream_t s) {
  const uint8_t* base = reinterpret_cast<const uint8_t*>(q.base);
  // kernel 1
  {
    Geo geo;
    geo.G = gcd_pow2_64(q.H / 32);
    geo.CPL = (q.H / 32) / geo.G;
    const int RPI = 64 / geo.G;
    const int RL = split ? kRLGateUpSplit<TM> : kRLGateUp<TM>;
    const int NI = RL * RPI / 2;
    const int tiles = (int)ceil_div(q.I, 4 * NI);
    const dim3 grid((unsigned)(max_active * tiles)), block(256);
    const auto kern = split ? ffn_gateup_kernel<BITS, TM, true, kRLGateUpSplit<TM>>
                            : ffn_gateup_kernel<BITS, TM, false, kRLGateUp<TM>>;
    launch_k(MOE_KERNEL_GEMV_GATEUP, kern, grid, block, 0, s, base, q.stride, q.slot_map, q.H, q.I, L.gate_codes,
             L.gate_sm, L.up_codes, L.up_sm, x, offsets, sorted_assign, active, n_active, k, tiles, geo, h_ws);
    if (moe_status st = check_launch("ffn_gateup")) return st;
  }
  // kernel 2
  {
    Geo geo;
    geo.G = gcd_pow2_64(q.I / 32);
    geo.CPL = (q.I / 32) / geo.G;
    const int RPI = 64 / geo.G;
    const int tiles = (int)ceil_div(q.H, 4 * kRLDown<TM> * RPI);
    const dim3 grid((unsigned)(max_active * tiles)), block(256);
    const auto kern = ybf16 ? ffn_down_kernel<BITS, TM, kRLDown<TM>, true> : ffn_down_kernel<BITS, TM, kRLDown<TM>, false>;
    launch_k(MOE_KERNEL_GEMV_DOWN, kern, grid, block, 0, s, base, q.stride, q.slot_map, q.H, q.I, L.down_codes,
             L.down_sm, h_ws, offsets, sorted_assign, active, n_active, tiles, geo, y);
    return check_launch("ffn_down");
  }
}

template <int BITS>
moe_status launch_bits(const moe_qlayer& q, const BlobLayout& L, const void* x, bool split, int T, int k,
                       const int32_t* offsets, const int32_t* sorted_assign, const int32_t* active,
                       const int32_t* n_active, int max_active, void* y, bool ybf16, float* h_ws, hipStream_t s) {
  if (T <= 1)
    return launch_bits_tm<BITS, 1>(q, L, x, split, k, offsets, sorted_assign, active, n_active, max_active, y, ybf16,
                                   h_ws, s);
  if (T <= 2)
    return launch_bits_tm<BITS, 2>(q, L, x, split, k, offsets, sorted_assign, active, n_active, max_active, y, ybf16,
                                   h_ws, s);
  return launch_bits_tm<BITS, 4>(q, L, x, split, k, offsets, sorted_assign, active, n_active, max_active, y, ybf16,
                                 h_ws, s);
}

}  // namespace

size_t ffn_gemv_ws_bytes(int n_assign, int I) { return (size_t)n_assign * (size_t)I * 4 + 256; }

moe_status launch_ffn_gemv(const moe_qlayer& q, const void* x, moe_dtype x_t, int T, int k, const int32_t* offsets,
                           const int32_t* sorted_assign, const int32_t* active, const int32_t* n_active, void* y,
                           moe_dtype y_t, void* ws, hipStream_t s) {
  const BlobLayout L = blob_layout(q.H, q.I, q.bits);
  const int max_active = (int)std::min<int64_t>(q.E, (int64_t)T * k);
  float* h_ws = reinterpret_cast<float*>(ws);
  const bool split = x_t == MOE_F32, ybf16 = y_t == MOE_BF16;
  if (q.bits == 2)
    return launch_bits<2>(q, L, x, split, T, k, offsets, sorted_assign, active, n_active, max_active, y, ybf16, h_ws,
                          s);
  return launch_bits<4>(q, L, x, split, T, k, offsets, sorted_assign, active, n_active, max_active, y, ybf16, h_ws, s);
}

}  // namespace moe
