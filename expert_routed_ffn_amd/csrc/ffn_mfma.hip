// ffn_mfma.hip -- expert FFN for prefill chunks: grouped GEMM on fp16 MFMA with
// fp32 accumulation.
//
// Passage: the prompt path reads up to 8,192 tokens per chunk (Strata feature,
// tech.hub77a.com, section "2. 왜 대단한가" (3)); reading a prompt touches all
// of the model's parameters (section "4. 해외 반응 쟁점"), so every expert gets
// many rows and the products become GEMMs.
//
// Per active expert e with n_e routed rows (sorted positions p0 .. p0+n_e):
//   gate/up:  C = X_e [n_e x H] * [Wg; Wu]^T  ->  h = silu(C_g) * C_u  (bf16)
//   down:     y = h [n_e x I] * Wd^T          ->  scattered to assignment rows
// Weights are decoded to half precision once per (tile, K-step) into LDS and
// fed to v_mfma_f32_16x16x32_f16 with fp32 accumulation.  One MFMA's K = 32 is
// one quantization block, so every K-step decodes one block per weight row.
//
// Rounding points: decoded weight = fp16_rne(fp32 fma(s, q, m)) for 2-bit
// codes and fp16_rne(s * q + m) (one fused fp16 operation) for 3- and 4-bit; x is
// converted to fp16 once by a pre-pass; h = silu(g) * u is rounded to fp16;
// products accumulate in fp32.
//
// Range.  The pre-pass scales each token row of x by a power of two 2^-e_t so
// that its largest magnitude lies in [1, 2) before the conversion; the gate and
// up accumulators of that token are then 2^-e_t times their true values, and h
// (quadratic in x for large gates) is kept as h' = h * 2^(-2 e_t) =
// g' * sigmoid(g' * 2^e_t) * u'.  The down epilogue multiplies by 2^(2 e_t).
// Power-of-two factors change no significant bit (outside fp16 subnormals), so
// the arithmetic is that of the unscaled values, without the fp16 range limit
// on x.  An h' beyond +-65504 (possible only for weights whose rows have an
// L1 norm far above the synthetic N(0, 0.02) ones) saturates and is counted in
// the first word of the workspace.  The operands are fp16 rather than bf16 because the
// weights' scale and min are fp16 values: fp16 keeps a decoded weight within
// 2^-12 of its exact value, bf16 only within 2^-9, and the bf16 rounding of the
// weights alone already moves outputs by 4e-3 to 9e-3 of their row maximum.
// Both types run at the same MFMA rate on gfx950.
//
// Two kernels.  mfma_rb_kernel (below, used when H % 256 == 0 and I % 128 ==
// 0) decodes each wave's weight rows straight into MFMA operand registers;
// mfma_ffn_kernel, described next, decodes the weight tile into LDS and serves
// every other shape.
//
// Tiling.  Workgroup = 4 waves in a 2 x 2 grid over a BM x BN output tile
// (128 x 256); each wave owns 64 x 128, i.e. 4 x 8 fragments of 16 x 16, so
// every fragment read from LDS feeds 4 to 8 MFMAs.  A wave's four 16-row
// groups are interleaved with the other wave row's, and groups past the
// tile's last row skip their MFMAs.  K-steps of 32 go through
// double-buffered LDS tiles (64-byte rows, 16-byte chunks permuted by row)
// with one barrier per step; global loads run two K-steps ahead, with no
// branch around them so that the compiler waits for one stage only.  When K
// is a multiple of 128 a thread fetches its B row's codes for two K-steps in
// one 16-byte buffer load (the pair pipeline), with the K-step offset in a
// scalar register.  Rows past a tile's end read an all-zero row kept after
// the last row of x16 and of h.  Workgroups are ordered so that the N-tiles of one M-tile run on the
// same die and share its L2 copy of the gathered activation rows.  The MFMAs take
// the weight fragment as their first operand, so the output comes transposed:
// a lane holds 4 consecutive columns of one row, stored as one 8- or 16-byte
// piece.  For gate/up the tile columns go in fours (gate i, gate i+1, up i,
// up i+1), so SwiGLU stays inside a lane and h leaves as packed pairs.
//
// 2-bit decode uses a 4-entry fp16 table per (row, block): the packed pair of
// codes (c_even, c_odd) in the two halfwords becomes a v_perm_b32 byte selector
// (2c, 2c+1 per halfword), i.e. ~2 VALU ops per weight; 4- and 3-bit codes
// decode in packed fp16 (see below), about 2.5 VALU ops per weight.
//
// A small prep kernel turns (n_active, active, offsets, slot map) into the
// list of M-tiles, each its expert's blob index, first sorted row and row
// count in one 16-byte entry, so a workgroup starts from one load instead of a
// chain of four; the GEMM grid is sized for the worst case and blocks past the
// list's end exit at once.
#include <type_traits>

#include "internal.hpp"

namespace moe {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kBK = 32;
constexpr int kXcd = 8;  // accelerator dies (each with its own L2) that workgroups are spread over
#ifndef MOE_MFMA_XCD_RANGE
#define MOE_MFMA_XCD_RANGE 1  // 0: interleaved, 1: die ranges for gate/up, 2: for both GEMMs
#endif
// LDS tile rows: 0 = 80-byte pitch (padded); 1, 2 = 64-byte pitch with the
// four 16-byte chunks of a row permuted by chunk ^ ((row >> SHIFT) & 3),
// SHIFT = 2 or 1.  Measured on gfx950 with 128-bit reads in the fragment
// pattern (lane & 15 = row, lane >> 4 = chunk): layout 2 runs at about 200
// bytes per clock per CU, layouts 0 and 1 at about 125; the row-per-lane
// stores of the B tile run at about 75 in layout 2 and 64 in layout 1.
#ifndef MOE_LDS_SWZ
#define MOE_LDS_SWZ 2
#endif
constexpr int kPitch = MOE_LDS_SWZ == 0 ? 40 : 32;  // fp16 elements per LDS row
__device__ __forceinline__ int lds_off(int row, int chunk) {  // fp16 offset of 16-byte chunk `chunk` of `row`
  if constexpr (MOE_LDS_SWZ == 0) return row * kPitch + chunk * 8;
  constexpr int SH = MOE_LDS_SWZ == 1 ? 2 : 1;
  return row * kPitch + ((chunk ^ ((row >> SH) & 3)) * 8);
}
constexpr float kF16Max = 65504.0f;
// Raw buffer resources: no range clamp (every access is in bounds by
// construction), default data format for 32-bit elements.
constexpr int kBufRecords = -1;
constexpr int kBufFlags = 0x00020000;


// Two floats -> packed fp16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const f16x2_t v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Saturate finite values to the fp16 range; NaN stays NaN.
__device__ __forceinline__ float sat_f16(float v) { return fabsf(v) > kF16Max ? copysignf(kF16Max, v) : v; }

// h' = g' * sigmoid(g' * 2^e) * u' with the hardware exp2 and reciprocal (each
// within about 1 ulp in fp32; h' is then rounded to fp16): exp(-z) overflows
// to +inf for large negative z, giving h' = -0, and underflows to 0 for large
// positive z, giving g' * u'; NaN stays NaN.
__device__ __forceinline__ float swiglu_scaled(float g, float u, int ex) {
  const float z = __builtin_amdgcn_ldexpf(g, ex);
  const float en = __builtin_amdgcn_exp2f(z * -1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + en) * u;
}
// The same with cz = -log2(e) * 2^e_t formed once per row: g * cz rounds
// exactly as (g * 2^e_t) * -log2(e) does, a power of two commuting with the
// rounding (barring overflow and subnormals).
__device__ __forceinline__ float swiglu_c(float g, float u, float cz) {
  const float en = __builtin_amdgcn_exp2f(g * cz);
  return g * __builtin_amdgcn_rcpf(1.0f + en) * u;
}

__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// 16 consecutive weights of one row-block half -> 8 packed fp16 pairs.
// BITS = 2: `code` holds 16 codes in one word (pair p at bits 2p / 16+2p).
__device__ __forceinline__ void decode16_b2(uint32_t code, uint32_t smw, uint32_t (&out)[8]) {
  const float s = f16lo(smw), m = f16hi(smw);
  const uint32_t lut_lo = pack_f16(__builtin_fmaf(s, 0.f, m), __builtin_fmaf(s, 1.f, m));
  const uint32_t lut_hi = pack_f16(__builtin_fmaf(s, 2.f, m), __builtin_fmaf(s, 3.f, m));
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t q2 = (code >> (2 * p)) & 0x00030003u;
    const uint32_t sel = q2 * 0x0202u + 0x01000100u;  // bytes (2q, 2q+1) for each halfword
    out[p] = __builtin_amdgcn_perm(lut_hi, lut_lo, sel);
  }
}

// 4- and 3-bit decode in packed fp16: a code pair (q_even, q_odd) or-ed into
// 0x6400 per halfword is the fp16 pair (1024 + q); subtracting 1024 is exact,
// and one fused multiply-add per pair gives fp16(s * q + m) with a single
// rounding.  About 5 VALU ops per pair against 10 through fp32.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}
struct Dec16 {  // the block's scale and min in both halfwords, and the -1024 pair
  f16x2_t s2, m2, off;
};
__device__ __forceinline__ Dec16 dec16(uint32_t smw) {
  Dec16 d;
  d.s2 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(smw, smw, 0x01000100u));
  d.m2 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(smw, smw, 0x03020302u));
  d.off = f16x2_t{(_Float16)-1024.0f, (_Float16)-1024.0f};
  return d;
}
__device__ __forceinline__ uint32_t dec_pair(uint32_t magic_pair, const Dec16& d) {
  const f16x2_t q = __builtin_bit_cast(f16x2_t, magic_pair) + d.off;
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, d.s2, d.m2));
}

// BITS = 4: two words, 8 codes each (pair p at bits 4p / 16+4p).
__device__ __forceinline__ void decode16_b4(uint32_t c0, uint32_t c1, uint32_t smw, uint32_t (&out)[8]) {
  const Dec16 d = dec16(smw);
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t c = w ? c1 : c0;
#pragma unroll
    for (int p = 0; p < 4; ++p) out[4 * w + p] = dec_pair(and_or(c >> (4 * p), 0x000F000Fu, 0x64006400u), d);
  }
}

// BITS = 3: `lo` holds the low two bits of 16 codes (pair p at bits 2p /
// 16+2p, as for 2 bits) and `hi` their high bits (pair p at bits p / 16+p).
__device__ __forceinline__ void decode16_b3(uint32_t lo, uint32_t hi, uint32_t smw, uint32_t (&out)[8]) {
  const Dec16 d = dec16(smw);
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t h2 = ((hi >> p) & 0x00010001u) << 2;
    out[p] = dec_pair(and_or(lo >> (2 * p), 0x00030003u, 0x64006400u | h2), d);
  }
}

struct TileInfo {  // one M-tile: its expert's blob index and its sorted rows p_begin .. p_begin + rows
  int32_t idx, p_begin, rows, pad;
};

// Build the M-tile list: for each active slot, ceil(n_e / BM) tiles.
__global__ __launch_bounds__(1024) void mfma_tiles_kernel(const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ active,
                                                          const int32_t* __restrict__ n_active,
                                                          const int32_t* __restrict__ slot_map, int BM,
                                                          TileInfo* __restrict__ tiles, int32_t* __restrict__ count) {
  __shared__ int sh[1024 / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int na = *n_active;
  int running = 0;
  for (int base = 0; base < na; base += 1024) {
    const int s = base + tid;
    int mt = 0, ne = 0, p0 = 0, idx = 0;
    if (s < na) {
      const int e = active[s];
      p0 = offsets[e];
      ne = offsets[e + 1] - p0;
      mt = (ne + BM - 1) / BM;
      idx = slot_map ? slot_map[e] : e;
    }
    int inc = mt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(inc, off, 64);
      if (lane >= off) inc += v;
    }
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < 1024 / 64; ++w) {
      if (w < wave) before += sh[w];
      total += sh[w];
    }
    const int start = running + before + inc - mt;
    for (int j = 0; j < mt; ++j) tiles[start + j] = TileInfo{idx, p0 + j * BM, min(BM, ne - j * BM), 0};
    running += total;
    __syncthreads();
  }
  if (tid == 0) *count = running;
}

// x [T x H] (bf16 bits or fp32) -> fp16 x * 2^-e_t (round to nearest even),
// one workgroup per row at a time: the row's largest magnitude m gives
// e_t = exponent of m (m * 2^-e_t in [1, 2)); a zero or non-finite m gives
// e_t = 0.  The exponents go to xexp [T].  Block 0 also clears the zero rows
// after x16 and h (z1, z2: 16-byte pieces) and the saturation counter.
template <bool XF32>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t i, float (&f)[8]) {
  if constexpr (XF32) {
    const float4 a = reinterpret_cast<const float4*>(x)[2 * i], b = reinterpret_cast<const float4*>(x)[2 * i + 1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  } else {
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = __uint_as_float(w[j] << 16);
      f[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
}

template <bool XF32>
__global__ __launch_bounds__(256) void to_f16_kernel(const void* __restrict__ x, int T, int H8,
                                                     uint4* __restrict__ out, int32_t* __restrict__ xexp,
                                                     uint4* __restrict__ z1, int n1, uint4* __restrict__ z2, int n2,
                                                     uint32_t* __restrict__ clip) {
  __shared__ float red[4];
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < n1; i += 256) z1[i] = make_uint4(0, 0, 0, 0);
    for (int i = threadIdx.x; i < n2; i += 256) z2[i] = make_uint4(0, 0, 0, 0);
    if (threadIdx.x == 0) *clip = 0;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    const int64_t r0 = (int64_t)t * H8;
    float mx = 0.f;
    for (int c = threadIdx.x; c < H8; c += 256) {
      float f[8];
      load8<XF32>(x, r0 + c, f);
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(f[j]));  // fmaxf drops NaN; +inf is kept
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();  // red is reused by the next row
    const int e = (mx > 0.f && mx <= 3.402823466e38f) ? __builtin_amdgcn_frexp_expf(mx) - 1 : 0;
    if (threadIdx.x == 0) xexp[t] = e;
    for (int c = threadIdx.x; c < H8; c += 256) {
      float f[8];
      load8<XF32>(x, r0 + c, f);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = __builtin_amdgcn_ldexpf(f[j], -e);
      out[r0 + c] = make_uint4(pack_f16(f[0], f[1]), pack_f16(f[2], f[3]), pack_f16(f[4], f[5]),
                               pack_f16(f[6], f[7]));
    }
  }
}

struct GemmArgs {
  const uint8_t* base;
  int64_t stride;
  int H, I, k;
  int64_t off_c0, off_s0, off_c1, off_s1;  // gate/up: Wg and Wu planes; down: Wd planes in c0/s0
  const _Float16* a_src;                   // x [T x H] (gate/up) or h [n x I] (down), fp16
  int64_t a_zero_row;                      // T or n: an all-zero row of a_src
  const int32_t* sorted_assign;
  const TileInfo* tiles;
  const int32_t* tile_count;
  int n_tiles_n;
  void* out;  // h [n x I] fp16 (gate/up) or y [T*k x H] (down)
  const int32_t* xexp;  // [T] the power-of-two exponent of each token row of x16
  uint32_t* clip;       // count of h values that saturated
};

// Two waves per SIMD (two workgroups per CU): the compiler keeps the 64 x 128
// accumulator tile of a wave in VGPRs within that budget.
// Activation rows loaded two K-steps at a time in the pair pipeline.
#ifndef MOE_MFMA_APAIR
#define MOE_MFMA_APAIR 1
#endif
#ifndef MOE_MFMA_WAVES_PER_EU
#define MOE_MFMA_WAVES_PER_EU 2
#endif
// NT threads = NT / 64 waves in a (NT / 128) x 2 grid over the BM x BN tile.
// PAIRB: the pair pipeline below (needs K a multiple of 128).
template <int BITS, int BM, int BN, bool GATEUP, bool YBF16, bool PAIRB, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(MOE_MFMA_WAVES_PER_EU))) void mfma_ffn_kernel(
    GemmArgs A) {
  constexpr int kBN = BN;
  constexpr int WMR = NT / 128;           // wave rows
  constexpr int FM = BM / (16 * WMR);     // 16-row fragments per wave
  constexpr int FN = BN / 32;             // 16-column fragments per wave
  constexpr int A_CHUNKS = BM * 4 / NT;   // 16-byte chunks of the A tile per thread per K-step
  constexpr int B_HALVES = 2 * BN / NT;   // 16-weight half rows of the B tile per thread per K-step
  static_assert(A_CHUNKS >= 1 && (B_HALVES == 1 || B_HALVES == 2), "tile and thread counts do not match");
  __shared__ __attribute__((aligned(16))) _Float16 lds_a[2][BM * kPitch];
  __shared__ __attribute__((aligned(16))) _Float16 lds_b[2][kBN * kPitch];

  // XCD-aware order: workgroups are handed to the kXcd dies round-robin by
  // index, so block b runs on die b % kXcd; the N-tiles of one M-tile are
  // given consecutive blocks on the same die, which then reads the M-tile's
  // activation rows into its own L2 once for all of them.
  const int xcd = blockIdx.x % kXcd, j = blockIdx.x / kXcd;
  int tile_idx, nt;
  if (MOE_MFMA_XCD_RANGE == 2 || (MOE_MFMA_XCD_RANGE == 1 && GATEUP)) {
    // Each die takes one contiguous range of the M-tile list (expert order),
    // so all M-tiles of an expert but those at a range boundary share one L2
    // for the expert's weights, as the N-tiles of an M-tile share it for the
    // activation rows.
    const int count = *A.tile_count, per_die = (count + kXcd - 1) / kXcd, jt = j / A.n_tiles_n;
    tile_idx = xcd * per_die + jt;
    nt = j % A.n_tiles_n;
    if (jt >= per_die || tile_idx >= count) return;
  } else {
    tile_idx = (j / A.n_tiles_n) * kXcd + xcd;
    nt = j % A.n_tiles_n;
    if (tile_idx >= *A.tile_count) return;
  }
  const TileInfo ti = A.tiles[tile_idx];  // one 16-byte load: no chain through active, offsets and the map
  const int p_begin = ti.p_begin, rows = ti.rows, idx = ti.idx;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = __builtin_amdgcn_readfirstlane(wave >> 1), wn = wave & 1;
  // Wave row wm owns the 16-row groups wm, wm + WMR, wm + 2 WMR, ... of the
  // tile (interleaved, so a partly filled tile loads the SIMDs evenly); its
  // first nv fragments hold rows of the tile, the rest are skipped.
  const int nv = max(0, min(FM, ((rows + 15) / 16 - wm + WMR - 1) / WMR));
  const int K = GATEUP ? A.H : A.I;
  const int KS = K / kBK;

  if (idx < 0) {  // expert not resident: NaN outputs, no weight reads
    const float nan = __builtin_nanf("");
    for (int c = tid; c < BM * kBN; c += NT) {
      const int m = c / kBN, col = c % kBN;
      if (m >= rows) continue;
      if constexpr (GATEUP) {
        const int g = col / 16, j = col % 16;
        const int i = nt * (kBN / 2) + 8 * g + j;
        if (j < 8 && i < A.I)
          reinterpret_cast<_Float16*>(A.out)[(size_t)(p_begin + m) * A.I + i] = (_Float16)nan;
      } else {
        const int n = nt * kBN + col;
        const int64_t a = A.sorted_assign[p_begin + m];
        if (n < A.H) {
          if constexpr (YBF16) reinterpret_cast<__bf16*>(A.out)[a * A.H + n] = (__bf16)nan;
          else reinterpret_cast<float*>(A.out)[a * A.H + n] = nan;
        }
      }
    }
    return;
  }
  const uint8_t* blob = A.base + (int64_t)idx * A.stride;

  // ---- A-tile sources: row pointer per chunk this thread copies --------------
  const uint8_t* a_row[A_CHUNKS];
  int a_col16[A_CHUNKS];
#pragma unroll
  for (int j = 0; j < A_CHUNKS; ++j) {
    const int c = tid + NT * j;
    const int m = c / 4;
    a_col16[j] = c % 4;
    // rows past the tile's end read the all-zero row kept after the last source row
    if constexpr (GATEUP) {
      const int64_t tok = m < rows ? A.sorted_assign[p_begin + m] / A.k : A.a_zero_row;
      a_row[j] = reinterpret_cast<const uint8_t*>(A.a_src + tok * (int64_t)A.H);
    } else {
      const int64_t p = m < rows ? p_begin + m : A.a_zero_row;
      a_row[j] = reinterpret_cast<const uint8_t*>(A.a_src + p * A.I);
    }
  }

  // ---- B-tile rows: tile row r -> weight row in its plane (rows past I or H
  // read row 0; their columns are never stored)
  const int64_t row_code_bytes = (int64_t)K * BITS / 8, row_sm_bytes = (int64_t)(K / 32) * 4;
  auto b_src = [&](int r, const uint8_t*& codes, const uint8_t*& sm) {
    int64_t row, oc, os;
    if constexpr (GATEUP) {
      // column 4q + j of 16-column group g: j = 0, 1 -> gate rows i, i + 1; j = 2, 3 -> up rows i, i + 1
      const int g = r / 16, q = (r % 16) / 4, jj = r % 4;
      const int i = nt * (kBN / 2) + 8 * g + 2 * q + (jj & 1);
      row = i < A.I ? i : 0;
      oc = jj < 2 ? A.off_c0 : A.off_c1;
      os = jj < 2 ? A.off_s0 : A.off_s1;
    } else {
      const int n = nt * kBN + r;
      row = n < A.H ? n : 0;
      oc = A.off_c0;
      os = A.off_s0;
    }
    codes = blob + oc + row * row_code_bytes;
    sm = blob + os + row * row_sm_bytes;
  };
  // this thread decodes B_HALVES x 16 weights of tile row b_r per K-step
  const int b_r = B_HALVES == 2 ? tid : tid >> 1, b_half0 = B_HALVES == 2 ? 0 : (tid & 1);
  const uint8_t* b_codes;
  const uint8_t* b_sm;
  b_src(b_r, b_codes, b_sm);

  // One K-step's global data, held in registers between its load and its LDS store.
  struct Stage {
    uint4 a[A_CHUNKS];
    uint32_t code[B_HALVES][BITS == 2 ? 1 : 2];
    uint32_t smw;
  };

  // Loads are unconditional (rows past the tile's end read a valid row whose
  // results are never stored), so every K-step issues the same loads and the
  // compiler can wait for one stage while later stages stay in flight.
  auto load_stage = [&](int ks) {
    Stage st;
#pragma unroll
    for (int jj = 0; jj < A_CHUNKS; ++jj)
      st.a[jj] = *reinterpret_cast<const uint4*>(a_row[jj] + (int64_t)ks * kBK * 2 + a_col16[jj] * 16);
#pragma unroll
    for (int hh = 0; hh < B_HALVES; ++hh) {
      const int b_half = b_half0 + hh;
      if constexpr (BITS == 2) {
        st.code[hh][0] = *reinterpret_cast<const uint32_t*>(b_codes + (int64_t)ks * 8 + b_half * 4);
      } else if constexpr (BITS == 3) {  // low bits of this half, then the block's high-bit word
        st.code[hh][0] = *reinterpret_cast<const uint32_t*>(b_codes + (int64_t)ks * 12 + b_half * 4);
        st.code[hh][1] = *reinterpret_cast<const uint32_t*>(b_codes + (int64_t)ks * 12 + 8) >> (8 * b_half);
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(b_codes + (int64_t)ks * 16 + b_half * 8);
        st.code[hh][0] = v.x;
        st.code[hh][1] = v.y;
      }
    }
    st.smw = *reinterpret_cast<const uint32_t*>(b_sm + (int64_t)ks * 4);
    return st;
  };

  // A chunks of one K-step into LDS buffer `buf`.
  auto store_a = [&](const uint4 (&a)[A_CHUNKS], int buf) {
#pragma unroll
    for (int jj = 0; jj < A_CHUNKS; ++jj) {
      const int c = tid + NT * jj;
      const int m = c / 4;
      *reinterpret_cast<uint4*>(&lds_a[buf][lds_off(m, a_col16[jj])]) = a[jj];
    }
  };
  // This thread's B slice of one K-step, decoded into LDS buffer `buf`.
  auto store_b = [&](const uint32_t (&code)[B_HALVES][BITS == 2 ? 1 : 2], uint32_t smw, int buf) {
#pragma unroll
    for (int hh = 0; hh < B_HALVES; ++hh) {
      uint32_t w[8];  // rows past I (or H) decode a valid row; their columns are never stored
      if constexpr (BITS == 2) decode16_b2(code[hh][0], smw, w);
      else if constexpr (BITS == 3) decode16_b3(code[hh][0], code[hh][1], smw, w);
      else decode16_b4(code[hh][0], code[hh][1], smw, w);
      const int c0 = 2 * (b_half0 + hh);
      *reinterpret_cast<uint4*>(&lds_b[buf][lds_off(b_r, c0)]) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(&lds_b[buf][lds_off(b_r, c0 + 1)]) = make_uint4(w[4], w[5], w[6], w[7]);
    }
  };
  auto store_stage = [&](const Stage st, int buf) {
    store_a(st.a, buf);
    store_b(st.code, st.smw, buf);
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int fi = 0; fi < FM; ++fi)
#pragma unroll
    for (int fj = 0; fj < FN; ++fj) acc[fi][fj] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int frag_r = lane & 15, frag_q = lane >> 4;  // row in the fragment, 16-byte chunk of K
  auto mma_stage = [&](int cur) {
    if (nv == 0) return;
    f16x8_t af[FM], bfr[FN];
#pragma unroll
    for (int fi = 0; fi < FM; ++fi)
      af[fi] = *reinterpret_cast<const f16x8_t*>(&lds_a[cur][lds_off(16 * (wm + WMR * fi) + frag_r, frag_q)]);
#pragma unroll
    for (int fj = 0; fj < FN; ++fj)
      bfr[fj] = *reinterpret_cast<const f16x8_t*>(&lds_b[cur][lds_off(wn * (BN / 2) + 16 * fj + frag_r, frag_q)]);
#pragma unroll
    for (int fi = 0; fi < FM; ++fi) {
      if (fi >= nv) break;
#pragma unroll
      for (int fj = 0; fj < FN; ++fj)
        acc[fi][fj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bfr[fj], af[fi], acc[fi][fj], 0, 0, 0);
    }
  };

  if constexpr (PAIRB) {
    {
      // Pair pipeline: the codes of a B row for two K-steps are one (2-bit) or
      // two (4-bit) 16-byte loads and their scale/min words one 8-byte load (the
      // two threads that share a row when NT = 2 BN load the same bytes).  Stage s sits in LDS
      // buffer s & 1; A runs two K-steps ahead in sa0/sa1 (even/odd stages), B
      // pairs in bp0 (stages 4j, 4j+1) and bp1 (4j+2, 4j+3); loads past the end
      // repeat the last K-step or pair and are never used.
      struct BPair {  // a row's codes for two K-steps (BITS words each) and both scale/min words
        uint32_t w[2 * BITS];
        uint2 sm;
      };
      // Buffer loads: a 32-bit per-lane offset from a workgroup-uniform base,
      // the K-step's offset in a scalar register (the host keeps every byte
      // offset below 2^31 for this kernel).
      const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<_Float16*>(A.a_src), (short)0, kBufRecords, kBufFlags);
      const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(blob), (short)0, kBufRecords, kBufFlags);
      const uint8_t* a_base = reinterpret_cast<const uint8_t*>(A.a_src);
      int a_voff[A_CHUNKS];
#pragma unroll
      for (int jj = 0; jj < A_CHUNKS; ++jj) a_voff[jj] = (int)(a_row[jj] - a_base) + a_col16[jj] * 16;
      const int bc_voff = (int)(b_codes - blob), bs_voff = (int)(b_sm - blob);
      auto load_a = [&](uint4 (&a)[A_CHUNKS], int ks) {
#pragma unroll
        for (int jj = 0; jj < A_CHUNKS; ++jj)
          a[jj] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsa, a_voff[jj], ks * kBK * 2, 0));
      };
      auto load_bpair = [&](BPair& bp, int ks) {  // ks even, ks + 1 < KS
        if constexpr (BITS == 3) {  // 24 bytes, 8-byte aligned: three 8-byte loads
#pragma unroll
          for (int j = 0; j < 3; ++j) {
            const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsb, bc_voff + 8 * j,
                                                                                             ks * (4 * BITS), 0));
            bp.w[2 * j] = v.x;
            bp.w[2 * j + 1] = v.y;
          }
        } else {
#pragma unroll
          for (int j = 0; j < BITS / 2; ++j) {
            const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsb, bc_voff + 16 * j,
                                                                                              ks * (4 * BITS), 0));
            bp.w[4 * j] = v.x;
            bp.w[4 * j + 1] = v.y;
            bp.w[4 * j + 2] = v.z;
            bp.w[4 * j + 3] = v.w;
          }
        }
        bp.sm = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsb, bs_voff, ks * 4, 0));
      };
      auto store_bpair = [&](const BPair& bp, int e, int buf) {  // e: which K-step of the pair
        // K-step e's words: 2-bit (half 0, half 1); 3-bit (low bits of half 0,
        // of half 1, high bits); 4-bit (two words per half)
        const uint32_t* c = bp.w + e * BITS;
        uint32_t code[B_HALVES][BITS == 2 ? 1 : 2];
#pragma unroll
        for (int hh = 0; hh < B_HALVES; ++hh) {
          const int h = B_HALVES == 2 ? hh : b_half0;  // two threads per row: each its half
          if constexpr (BITS == 2) {
            code[hh][0] = h ? c[1] : c[0];
          } else if constexpr (BITS == 3) {
            code[hh][0] = h ? c[1] : c[0];
            code[hh][1] = h ? c[2] >> 8 : c[2];
          } else {
            code[hh][0] = h ? c[2] : c[0];
            code[hh][1] = h ? c[3] : c[1];
          }
        }
        store_b(code, e ? bp.sm.y : bp.sm.x, buf);
      };
#if MOE_MFMA_APAIR
      // A in pairs as well: a00/a01 hold stages 4j, 4j+1 and a10/a11 stages
      // 4j+2, 4j+3; both K-steps of a pair are loaded back to back, so the
      // second 64-byte half of each activation line is requested while the
      // first is still in flight.
      uint4 a00[A_CHUNKS], a01[A_CHUNKS], a10[A_CHUNKS], a11[A_CHUNKS];
      BPair bp0, bp1;
      load_a(a00, 0);
      load_a(a01, 1);
      load_a(a10, 2);
      load_a(a11, 3);
      load_bpair(bp0, 0);
      load_bpair(bp1, 2);
      store_a(a00, 0);
      store_bpair(bp0, 0, 0);
      __syncthreads();
      for (int kb = 0; kb < KS; kb += 4) {
        mma_stage(0);  // stage kb
        __builtin_amdgcn_sched_barrier(0);  // the decode below starts after the MFMAs are issued
        store_a(a01, 1);
        store_bpair(bp0, 1, 1);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);  // keep each K-step's loads and MFMAs in their own step
        load_a(a00, min(kb + 4, KS - 1));
        load_a(a01, min(kb + 5, KS - 1));
        load_bpair(bp0, min(kb + 4, KS - 2));
        mma_stage(1);  // stage kb + 1
        __builtin_amdgcn_sched_barrier(0);
        store_a(a10, 0);
        store_bpair(bp1, 0, 0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        mma_stage(0);  // stage kb + 2
        __builtin_amdgcn_sched_barrier(0);
        store_a(a11, 1);
        store_bpair(bp1, 1, 1);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        load_a(a10, min(kb + 6, KS - 1));
        load_a(a11, min(kb + 7, KS - 1));
        load_bpair(bp1, min(kb + 6, KS - 2));
        mma_stage(1);  // stage kb + 3
        __builtin_amdgcn_sched_barrier(0);
        store_a(a00, 0);
        store_bpair(bp0, 0, 0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
#else
      uint4 sa0[A_CHUNKS], sa1[A_CHUNKS];
      BPair bp0, bp1;
      load_a(sa0, 0);
      load_a(sa1, 1);
      load_bpair(bp0, 0);
      load_bpair(bp1, 2);
      store_a(sa0, 0);
      store_bpair(bp0, 0, 0);
      __syncthreads();
      for (int kb = 0; kb < KS; kb += 4) {
        load_a(sa0, min(kb + 2, KS - 1));
        mma_stage(0);  // stage kb
        __builtin_amdgcn_sched_barrier(0);  // the decode below starts after the MFMAs are issued
        store_a(sa1, 1);
        store_bpair(bp0, 1, 1);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);  // keep each K-step's loads and MFMAs in their own step
        load_a(sa1, min(kb + 3, KS - 1));
        load_bpair(bp0, min(kb + 4, KS - 2));
        mma_stage(1);  // stage kb + 1
        __builtin_amdgcn_sched_barrier(0);  // the decode below starts after the MFMAs are issued
        store_a(sa0, 0);
        store_bpair(bp1, 0, 0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);  // keep each K-step's loads and MFMAs in their own step
        load_a(sa0, min(kb + 4, KS - 1));
        mma_stage(0);  // stage kb + 2
        __builtin_amdgcn_sched_barrier(0);  // the decode below starts after the MFMAs are issued
        store_a(sa1, 1);
        store_bpair(bp1, 1, 1);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);  // keep each K-step's loads and MFMAs in their own step
        load_a(sa1, min(kb + 5, KS - 1));
        load_bpair(bp1, min(kb + 6, KS - 2));
        mma_stage(1);  // stage kb + 3
        __builtin_amdgcn_sched_barrier(0);  // the decode below starts after the MFMAs are issued
        store_a(sa0, 0);
        store_bpair(bp0, 0, 0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);  // keep each K-step's loads and MFMAs in their own step
      }
#endif
    }
  } else {
    // Software pipeline: global loads run two K-steps ahead of the MFMAs
    // (even stages in s0, odd in s1, from the load to the LDS store); LDS is
    // double-buffered, one barrier per K-step.  No load sits behind a branch:
    // stages past the end reload the last K-step (never used), so a store
    // waits only for its own stage.
    Stage s0 = load_stage(0), s1 = load_stage(min(1, KS - 1));
    store_stage(s0, 0);
    __syncthreads();
    for (int kb = 0; kb < KS; kb += 2) {
      s0 = load_stage(min(kb + 2, KS - 1));  // s0 held stage kb, already in LDS
      mma_stage(0);
      store_stage(s1, 1);
      __syncthreads();
      s1 = load_stage(min(kb + 3, KS - 1));
      if (kb + 1 < KS) mma_stage(1);
      store_stage(s0, 0);
      __syncthreads();
    }
  }


  // ---- epilogue.  The MFMAs take the weights as their first operand, so a
  // lane holds 4 consecutive output columns of one row: row 16 * fi + (lane & 15),
  // columns 16 * fj + 4 * (lane >> 4) + r.
  const int frow = lane & 15, fcol = 4 * (lane >> 4);
#pragma unroll
  for (int fi = 0; fi < FM; ++fi) {
    const int m = 16 * (wm + WMR * fi) + frow;
    if (m >= rows) continue;
    if constexpr (GATEUP) {
      // columns 4q .. 4q + 3 = gate i, gate i + 1, up i, up i + 1, all 2^-e_t
      // times their true values: h' = g' * sigmoid(g' * 2^e_t) * u' = h * 2^(-2 e_t)
      _Float16* hrow = reinterpret_cast<_Float16*>(A.out) + (size_t)(p_begin + m) * A.I;
      const int ex = A.xexp[A.sorted_assign[p_begin + m] / A.k];
      int sat = 0;
#pragma unroll
      for (int fj = 0; fj < FN; ++fj) {
        const int i = nt * (kBN / 2) + 8 * (FN * wn + fj) + fcol / 2;
        if (i >= A.I) continue;
        const f32x4_t v = acc[fi][fj];
        const float h0 = swiglu_scaled(v[0], v[2], ex);
        const float h1 = swiglu_scaled(v[1], v[3], ex);
        sat += (fabsf(h0) > kF16Max) + (fabsf(h1) > kF16Max);
        *reinterpret_cast<uint32_t*>(hrow + i) = pack_f16(sat_f16(h0), sat_f16(h1));
      }
      if (sat) atomicAdd(A.clip, (uint32_t)sat);
    } else {
      const int64_t a = A.sorted_assign[p_begin + m];
      const int ey = 2 * A.xexp[a / A.k];
#pragma unroll
      for (int fj = 0; fj < FN; ++fj) {
        const int n = nt * kBN + wn * (BN / 2) + 16 * fj + fcol;
        if (n >= A.H) continue;
        f32x4_t v = acc[fi][fj];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = __builtin_amdgcn_ldexpf(v[r], ey);
        if constexpr (YBF16) {
          const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[0]) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[1]) << 16);
          const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2]) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[3]) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<__bf16*>(A.out) + a * A.H + n) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(A.out) + a * A.H + n) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
}

// ---- weights decoded into registers (32 x 32 x 16 MFMA) ------------------------
// The same GEMMs with the decoded weight tile never in LDS.  Each of the 4
// waves owns 64 of the tile's 256 weight rows for all 128 tile rows: 4 x 2
// fragments of v_mfma_f32_32x32x16_f16 (weights as the first operand:
// D[n][t]).  A lane supplies 8 K-values of one weight row per MFMA, so it
// decodes those weights itself, straight into the operand registers, from its
// row's code words and scale/min word; no two waves decode the same row.  The
// raw codes and scale/min words reach LDS in 4-K-step chunks loaded as whole
// 16-byte pieces of each row (half the cache-line accesses of per-lane
// loads), stored K-step-major; the activation tile goes through LDS as
// before (8 KB per K-step).  Weight rows are placed so that a lane's 16
// outputs of a fragment are 8 consecutive h columns (gate/up: gate and up of
// each i in the same lane) or 16 consecutive y columns (down): one 16-byte
// store per 8 values.
//
// Operand layouts (32 x 32 x 16, f16): lane l gives row l % 32 of the first
// operand and column l % 32 of the second, K-values 8 (l / 32) .. + 8 of the
// 16; it receives D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32] in accumulator v.
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Activation tile rows (64 bytes) with chunk c stored at c ^ ((row >> 2) & 3):
// the fragment reads (32 consecutive rows, one chunk per half-wave) then touch
// each bank once per 16 lanes.
__device__ __forceinline__ int lds_off_rb(int row, int chunk) { return row * kPitch + ((chunk ^ ((row >> 2) & 3)) * 8); }

// Codes decoded in place: the pair of codes at bits p / 16 + p (mask: the
// code's bits at 0 / 16) is masked out of the word unshifted and ORed into
// fp16 2^(10 - p), whose mantissa bit p is worth 1, so each half reads
// 2^(10 - p) + q exactly (p + code width <= 10); subtracting 2^(10 - p)
// leaves q, and one packed fma gives fp16(s q + m) with a single rounding.
template <int P, uint32_t MASK>
__device__ __forceinline__ uint32_t dec_pair_at(uint32_t w, const Dec16& d) {
  static_assert(P >= 0 && P <= 10, "code inside the fp16 mantissa");
  constexpr uint32_t e = 0x6400u - 0x0400u * P;  // fp16 bits of 2^(10 - P)
  const _Float16 base = __builtin_bit_cast(_Float16, (uint16_t)e);
  const f16x2_t q = __builtin_bit_cast(f16x2_t, and_or(w, MASK << P, e | (e << 16))) - f16x2_t{base, base};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, d.s2, d.m2));
}

// 3-bit codes in place: pair J's low bits at 2J / 16 + 2J of `lo`, its high
// bits at J / 16 + J of `hi`; hi << (J + 2) puts them at 2J + 2, above the
// low bits, and the three bits decode as in dec_pair_at with p = 2J.
template <int J>
__device__ __forceinline__ uint32_t dec_pair3_at(uint32_t lo, uint32_t hi, const Dec16& d) {
  constexpr int P = 2 * J;
  constexpr uint32_t e = 0x6400u - 0x0400u * P;  // fp16 bits of 2^(10 - P)
  const _Float16 base = __builtin_bit_cast(_Float16, (uint16_t)e);
  const uint32_t t = and_or(hi << (J + 2), 0x00040004u << P, e | (e << 16));
  const f16x2_t q = __builtin_bit_cast(f16x2_t, and_or(lo, 0x00030003u << P, t)) - f16x2_t{base, base};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, d.s2, d.m2));
}

// 8 weights (4 packed pairs) of one row for K-half kh of a K-step, lane half
// hh = l / 32 (weights 16 kh + 8 hh .. + 8 of the block).  c: the K-step's code
// words (2-bit: one per 16 weights; 3-bit: low bits of each half, then the
// high-bit word; 4-bit: two per 16 weights).
template <int BITS>
__device__ __forceinline__ void dec8(const uint32_t* c, int kh, int hh, const Dec16& d, uint32_t (&o)[4]) {
  if constexpr (BITS == 2) {
    const uint32_t w = c[kh] >> (8 * hh);  // pairs 4 hh .. 4 hh + 3 at bits 2j / 16 + 2j
    o[0] = dec_pair_at<0, 0x00030003u>(w, d);
    o[1] = dec_pair_at<2, 0x00030003u>(w, d);
    o[2] = dec_pair_at<4, 0x00030003u>(w, d);
    o[3] = dec_pair_at<6, 0x00030003u>(w, d);
  } else if constexpr (BITS == 3) {
    const uint32_t lo = c[kh] >> (8 * hh), hi = (c[2] >> (8 * kh)) >> (4 * hh);
    o[0] = dec_pair3_at<0>(lo, hi, d);
    o[1] = dec_pair3_at<1>(lo, hi, d);
    o[2] = dec_pair3_at<2>(lo, hi, d);
    o[3] = dec_pair3_at<3>(lo, hi, d);
  } else {
    const uint32_t w = hh ? c[2 * kh + 1] : c[2 * kh], w8 = w >> 8;  // pairs at bits 4j / 16 + 4j
    o[0] = dec_pair_at<0, 0x000F000Fu>(w, d);
    o[1] = dec_pair_at<4, 0x000F000Fu>(w, d);
    o[2] = dec_pair_at<0, 0x000F000Fu>(w8, d);
    o[3] = dec_pair_at<4, 0x000F000Fu>(w8, d);
  }
}

template <int BITS, bool GATEUP, bool YBF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mfma_rb_kernel(GemmArgs A) {
  constexpr int BM = 128, BN = 256, NT = 256, A_CHUNKS = 2;
  __shared__ __attribute__((aligned(16))) _Float16 lds_a[2][BM * kPitch];
  __shared__ __attribute__((aligned(16))) uint32_t lds_bc[2][4][BN * BITS];  // [buffer][K-step][row, word]
  __shared__ __attribute__((aligned(16))) uint32_t lds_bs[2][4][BN];         // [buffer][K-step][row]

  const int xcd = blockIdx.x % kXcd, jb = blockIdx.x / kXcd;
  int tile_idx, nt;
  if (MOE_MFMA_XCD_RANGE == 2 || (MOE_MFMA_XCD_RANGE == 1 && GATEUP)) {
    const int count = *A.tile_count, per_die = (count + kXcd - 1) / kXcd, jt = jb / A.n_tiles_n;
    tile_idx = xcd * per_die + jt;
    nt = jb % A.n_tiles_n;
    if (jt >= per_die || tile_idx >= count) return;
  } else {
    tile_idx = (jb / A.n_tiles_n) * kXcd + xcd;
    nt = jb % A.n_tiles_n;
    if (tile_idx >= *A.tile_count) return;
  }
  const TileInfo ti = A.tiles[tile_idx];  // one 16-byte load: no chain through active, offsets and the map
  const int p_begin = ti.p_begin, rows = ti.rows, idx = ti.idx;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, jl = lane & 31;
  const int nv = (rows + 31) / 32;  // 32-row fragments holding rows of the tile
  const int K = GATEUP ? A.H : A.I;
  const int KS = K / kBK;

  if (idx < 0) {  // expert not resident: NaN outputs, no weight reads
    const float nan = __builtin_nanf("");
    constexpr int COLS = GATEUP ? BN / 2 : BN;
    for (int c = tid; c < BM * COLS; c += NT) {
      const int m = c / COLS, col = c % COLS;
      if (m >= rows) continue;
      if constexpr (GATEUP) {
        reinterpret_cast<_Float16*>(A.out)[(size_t)(p_begin + m) * A.I + nt * COLS + col] = (_Float16)nan;
      } else {
        const int64_t a = A.sorted_assign[p_begin + m];
        if constexpr (YBF16) reinterpret_cast<__bf16*>(A.out)[a * A.H + nt * COLS + col] = (__bf16)nan;
        else reinterpret_cast<float*>(A.out)[a * A.H + nt * COLS + col] = nan;
      }
    }
    return;
  }
  const uint8_t* blob = A.base + (int64_t)idx * A.stride;

  // The epilogue's row information, fetched under the K-loop: thread t < rows
  // holds tile row t's assignment (issued here) and its token's exponent
  // (issued after the loop's first barrier, when the assignment has arrived),
  // handed to the lanes of that row through LDS after the loop.
  const bool ri_on = tid < BM && tid < rows;
  int ri_a = 0, ri_e = 0;
  if (ri_on) ri_a = A.sorted_assign[p_begin + tid];

  // ---- activation tile: two 16-byte chunks per thread per K-step ----------------
  int a_voff[A_CHUNKS], a_lds[A_CHUNKS];
#pragma unroll
  for (int jj = 0; jj < A_CHUNKS; ++jj) {
    const int c = tid + NT * jj, m = c / 4, ch = c % 4;
    int64_t row;  // rows past the tile's end read the all-zero row kept after the last source row
    if constexpr (GATEUP) row = m < rows ? A.sorted_assign[p_begin + m] / A.k : A.a_zero_row;
    else row = m < rows ? p_begin + m : A.a_zero_row;
    a_voff[jj] = (int)(row * (int64_t)K * 2) + ch * 16;
    a_lds[jj] = lds_off_rb(m, ch);
  }

  // ---- weight rows -------------------------------------------------------------
  // Tile weight row R = 64 wave + 32 fn + j holds fragment row j of wave
  // `wave`'s fragment fn; j = 8 g + 4 hb + r (g < 4, hb < 2, r < 4) is
  //   gate/up: plane r >> 1 (gate, up), i = nt*128 + 32*wave + 16*fn + 8*hb + 2*g + (r & 1)
  //   down:    n = nt*256 + 64*wave + 32*fn + 16*hb + 4*g + r
  // (rows past I or H read row 0; their outputs are never stored).
  const int64_t row_code_bytes = (int64_t)K * BITS / 8, row_sm_bytes = (int64_t)(K / 32) * 4;
  auto row_offsets = [&](int R, int& code_off, int& sm_off) {
    const int w = R >> 6, fn = (R >> 5) & 1, j = R & 31;
    const int g = j >> 3, hb = (j >> 2) & 1, r = j & 3;
    int64_t row, oc, os;
    if constexpr (GATEUP) {
      const int i = nt * (BN / 2) + 32 * w + 16 * fn + 8 * hb + 2 * g + (r & 1);
      row = i < A.I ? i : 0;
      oc = (r >> 1) ? A.off_c1 : A.off_c0;
      os = (r >> 1) ? A.off_s1 : A.off_s0;
    } else {
      const int n = nt * BN + 64 * w + 32 * fn + 16 * hb + 4 * g + r;
      row = n < A.H ? n : 0;
      oc = A.off_c0;
      os = A.off_s0;
    }
    code_off = (int)(oc + row * row_code_bytes);
    sm_off = (int)(os + row * row_sm_bytes);
  };
  // The weight codes and scale/min words go through LDS in chunks of 4
  // K-steps: each row's 16 BITS bytes of codes and 16 bytes of scale/min per
  // chunk are loaded as whole 16-byte pieces (consecutive threads on
  // consecutive pieces of a row) and stored K-step-major, [K-step][row], so a
  // wave's 32 rows of one K-step are one contiguous run when the lanes read
  // their own row's words.  Thread t loads code pieces t + 256 i (i < BITS) and
  // the scale/min piece of row t.
  constexpr int CK = 4;
  int bc_goff[BITS], bc_row[BITS], bc_piece[BITS], bs_goff;
#pragma unroll
  for (int i = 0; i < BITS; ++i) {
    const int pc = tid + NT * i;
    bc_row[i] = pc / BITS;
    bc_piece[i] = pc % BITS;
    int co, so;
    row_offsets(bc_row[i], co, so);
    bc_goff[i] = co + 16 * bc_piece[i];
  }
  {
    int co;
    row_offsets(tid, co, bs_goff);
  }
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(A.a_src), (short)0, kBufRecords, kBufFlags);
  const __amdgpu_buffer_rsrc_t rsb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blob), (short)0, kBufRecords, kBufFlags);

  struct BStage {  // this thread's pieces of one chunk
    uint4 c[BITS];
    uint4 s;
  };
  struct BStep {  // one K-step of this lane's two rows: codes and scale/min word
    uint32_t w[2][BITS];
    uint32_t sm[2];
  };
  auto load_a = [&](uint4 (&a)[A_CHUNKS], int ks) {
#pragma unroll
    for (int jj = 0; jj < A_CHUNKS; ++jj)
      a[jj] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsa, a_voff[jj], ks * kBK * 2, 0));
  };
  auto store_a = [&](const uint4 (&a)[A_CHUNKS], int buf) {
#pragma unroll
    for (int jj = 0; jj < A_CHUNKS; ++jj) *reinterpret_cast<uint4*>(&lds_a[buf][a_lds[jj]]) = a[jj];
  };
  auto load_bchunk = [&](BStage& st, int kc) {  // kc: the chunk's first K-step, kc + CK <= KS
#pragma unroll
    for (int i = 0; i < BITS; ++i)
      st.c[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsb, bc_goff[i], kc * (4 * BITS), 0));
    st.s = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsb, bs_goff, kc * 4, 0));
  };
  auto store_bchunk = [&](const BStage& st, int buf) {
#pragma unroll
    for (int i = 0; i < BITS; ++i) {
      const uint32_t v[4] = {st.c[i].x, st.c[i].y, st.c[i].z, st.c[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int wi = 4 * bc_piece[i] + q;  // word of the row's chunk: K-step wi / BITS, word wi % BITS
        lds_bc[buf][wi / BITS][bc_row[i] * BITS + wi % BITS] = v[q];
      }
    }
    lds_bs[buf][0][tid] = st.s.x;
    lds_bs[buf][1][tid] = st.s.y;
    lds_bs[buf][2][tid] = st.s.z;
    lds_bs[buf][3][tid] = st.s.w;
  };
  auto read_bstep = [&](BStep& bs, int buf, int ksl) {
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) {
      const int R = 64 * wave + 32 * fn + jl;
#pragma unroll
      for (int w = 0; w < BITS; ++w) bs.w[fn][w] = lds_bc[buf][ksl][R * BITS + w];
      bs.sm[fn] = lds_bs[buf][ksl][R];
    }
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;

  // ---- the K-step pieces -------------------------------------------------------
  auto tables = [&](const BStep& bs, Dec16 (&d)[2]) {
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) d[fn] = dec16(bs.sm[fn]);
  };
  auto dec_half = [&](const BStep& bs, int kh, const Dec16 (&d)[2], f16x8_t (&bo)[2]) {
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) {
      uint32_t o[4];
      dec8<BITS>(bs.w[fn], kh, hh, d[fn], o);
      bo[fn] = __builtin_bit_cast(f16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
    }
  };
  // Activation operands of K-half kh from LDS buffer `cur`.
  auto read_a = [&](int cur, int kh, f16x8_t (&ao)[4]) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
      ao[fm] = *reinterpret_cast<const f16x8_t*>(&lds_a[cur][lds_off_rb(32 * fm + jl, 2 * kh + hh)]);
  };
  // The MFMAs of one K-half over the first NV fragment rows (NV = 0: the
  // first nv, a runtime count), then `work` (the next operands' loads from LDS
  // and decode), which the compiler schedules in between the MFMAs when NV is
  // fixed.  Pinning that interleave (one MFMA, then up to five vector
  // instructions) measured 2.5% slower on the 2-bit gate/up GEMM.
  auto mfma_half = [&](auto nvc, const f16x8_t (&bo)[2], const f16x8_t (&ao)[4], auto&& work) {
    constexpr int NV = decltype(nvc)::value;
    if constexpr (NV == 0) {
#pragma unroll
      for (int fm = 0; fm < 4; ++fm) {
        if (fm >= nv) break;
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bo[fn], ao[fm], acc[fm][fn], 0, 0, 0);
      }
      work();
    } else {
#pragma unroll
      for (int fm = 0; fm < NV; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bo[fn], ao[fm], acc[fm][fn], 0, 0, 0);
      work();
    }
  };

  // Pipeline: activation chunks two K-steps ahead in registers (sa0 even
  // stages, sa1 odd), LDS double-buffered with one barrier per K-step; weight
  // chunks (4 K-steps) loaded into registers three K-steps before they are
  // stored to their LDS buffer (double-buffered, stored one K-step before
  // their first use).  A K-half's operands (activation fragments and this
  // lane's weight words from LDS, weights decoded) are prepared under the
  // MFMAs of the K-half before.  For 2- and 4-bit codes the loop is
  // specialised on the number of filled fragment rows (nv), so that it has no
  // branch but the loop's own and the scheduler can interleave the decode
  // with the MFMAs.
  // Loads past the end repeat the last K-step or chunk and are never used.
  auto run = [&](auto nvc) {
    uint4 sa0[A_CHUNKS], sa1[A_CHUNKS];
    BStage st;
    load_a(sa0, 0);
    load_a(sa1, min(1, KS - 1));
    load_bchunk(st, 0);
    store_a(sa0, 0);
    store_bchunk(st, 0);
    __syncthreads();
    if (ri_on) ri_e = A.xexp[ri_a / A.k];
    load_a(sa0, min(2, KS - 1));
    load_bchunk(st, min(CK, KS - CK));
    f16x8_t ao0[4], ao1[4], bo[2], bo2[2];
    Dec16 d[2] = {};
    BStep cs, ns;
    read_a(0, 0, ao0);
    read_bstep(cs, 0, 0);
    tables(cs, d);
    dec_half(cs, 0, d, bo);
    __builtin_amdgcn_sched_barrier(0);
    // One K-step (activation buffer `buf`); the next K-step's weights are
    // K-step nksl of weight buffer nbb; `pre` runs before the barrier.
    auto step = [&](int buf, int nbb, int nksl, const uint4 (&a_next)[A_CHUNKS], auto&& pre) {
      mfma_half(nvc, bo, ao0, [&] {
        read_a(buf, 1, ao1);
        read_bstep(ns, nbb, nksl);
        dec_half(cs, 1, d, bo2);
      });
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(nvc, bo2, ao1, [&] {
        tables(ns, d);
        dec_half(ns, 0, d, bo);
      });
      __builtin_amdgcn_sched_barrier(0);
      store_a(a_next, buf ^ 1);
      pre();
      __syncthreads();
      read_a(buf ^ 1, 0, ao0);
      cs = ns;
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int kb = 0; kb < KS; kb += 4) {
      const int bb = (kb / CK) & 1;
      step(0, bb, 1, sa1, [] {});  // stage kb (sa1: stage kb + 1)
      load_a(sa1, min(kb + 3, KS - 1));
      __builtin_amdgcn_sched_barrier(0);
      step(1, bb, 2, sa0, [] {});  // stage kb + 1 (sa0: stage kb + 2)
      load_a(sa0, min(kb + 4, KS - 1));
      __builtin_amdgcn_sched_barrier(0);
      step(0, bb, 3, sa1, [&] { store_bchunk(st, bb ^ 1); });  // stage kb + 2; the next chunk into LDS
      load_a(sa1, min(kb + 5, KS - 1));
      __builtin_amdgcn_sched_barrier(0);
      step(1, bb ^ 1, 0, sa0, [] {});  // stage kb + 3
      load_a(sa0, min(kb + 6, KS - 1));
      load_bchunk(st, min(kb + 2 * CK, KS - CK));
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if constexpr (BITS != 3) {  // the specialised loops spill for 3-bit codes
    switch (nv) {
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      default: run(std::integral_constant<int, 4>{}); break;
    }
  } else {
    run(std::integral_constant<int, 0>{});
  }

  // ---- epilogue: lane holds token row 32 fm + lane % 32 of the tile ----------------
  __syncthreads();  // every wave is past its last activation reads
  int2* lds_ri = reinterpret_cast<int2*>(&lds_a[0][0]);
  if (ri_on) lds_ri[tid] = make_int2(ri_a, ri_e);
  __syncthreads();
#pragma unroll
  for (int fm = 0; fm < 4; ++fm) {
    const int m = 32 * fm + jl;
    if (fm >= nv || m >= rows) continue;
    const int2 ri = lds_ri[m];  // (assignment, token exponent) of row m
    if constexpr (GATEUP) {
      // accumulator 4 g + s: gate of i = base + 2 g + s; 4 g + 2 + s: its up (s = 0, 1); all
      // 2^-e_t times their true values: h' = g' * sigmoid(g' * 2^e_t) * u' = h * 2^(-2 e_t)
      _Float16* hrow = reinterpret_cast<_Float16*>(A.out) + (size_t)(p_begin + m) * A.I;
      const float cz = __builtin_amdgcn_ldexpf(-1.4426950408889634f, ri.y);  // -log2(e) 2^e_t, exact
      float h[2][8], mx = 0.f;
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t& v = acc[fm][fn];
          h[fn][2 * g] = swiglu_c(v[4 * g], v[4 * g + 2], cz);
          h[fn][2 * g + 1] = swiglu_c(v[4 * g + 1], v[4 * g + 3], cz);
          mx = fmaxf(mx, fmaxf(fabsf(h[fn][2 * g]), fabsf(h[fn][2 * g + 1])));
        }
      if (mx > kF16Max) {  // rare: count the values past fp16 range and clamp them
        int sat = 0;
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            sat += fabsf(h[fn][q]) > kF16Max;
            h[fn][q] = sat_f16(h[fn][q]);
          }
        atomicAdd(A.clip, (uint32_t)sat);
      }
#pragma unroll
      for (int fn = 0; fn < 2; ++fn) {
        const int i0 = nt * (BN / 2) + 32 * wave + 16 * fn + 8 * hh;
        *reinterpret_cast<uint4*>(hrow + i0) =
            make_uint4(pack_f16(h[fn][0], h[fn][1]), pack_f16(h[fn][2], h[fn][3]), pack_f16(h[fn][4], h[fn][5]),
                       pack_f16(h[fn][6], h[fn][7]));
      }
    } else {
      const int64_t a = ri.x;
      const int ey = 2 * ri.y;
#pragma unroll
      for (int fn = 0; fn < 2; ++fn) {
        const int n0 = nt * BN + 64 * wave + 32 * fn + 16 * hh;
        f32x16_t v = acc[fm][fn];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = __builtin_amdgcn_ldexpf(v[r], ey);
        if constexpr (YBF16) {
          uint32_t pk[8];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            pk[q] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2 * q]) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2 * q + 1]) << 16);
          uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(A.out) + a * A.H + n0);
          dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
          dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
        } else {
          float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(A.out) + a * A.H + n0);
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
      }
    }
  }
}

// 128 x 256 tiles with 256 threads (two workgroups per CU).  256 x 256 tiles
// with 512 threads share one decoded B tile between twice the rows (a third
// fewer M-tiles on the prefill workload) but measured no faster.
#ifndef MOE_MFMA_BM
#define MOE_MFMA_BM 128
#endif
#ifndef MOE_MFMA_BN_GU
#define MOE_MFMA_BN_GU 256
#endif
#ifndef MOE_MFMA_BN_DN
#define MOE_MFMA_BN_DN 256
#endif
#ifndef MOE_MFMA_REGB
#define MOE_MFMA_REGB 1
#endif
constexpr bool kRegB = MOE_MFMA_REGB != 0;
constexpr int kBM = MOE_MFMA_BM;
constexpr int kBNGateUp = MOE_MFMA_BN_GU;
constexpr int kBNDown = MOE_MFMA_BN_DN;
constexpr int kNT = 2 * kBM;  // one wave per 64 x 128 piece of the tile

struct MfmaWs {
  uint32_t* clip;
  _Float16* x16;
  _Float16* h;
  TileInfo* tiles;
  int32_t* count;
  int32_t* xexp;
  size_t bytes;
};

MfmaWs carve(uint8_t* ws, int T, int H, int n, int E, int I) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const int max_tiles = (int)ceil_div(n, kBM) + std::min(E, n);
  MfmaWs w;
  size_t off = 0;
  w.clip = reinterpret_cast<uint32_t*>(ws + off);  // first word: the saturation count
  off += 256;
  w.x16 = reinterpret_cast<_Float16*>(ws + off);  // T rows, then one row of zeros
  off += up((size_t)(T + 1) * H * 2);
  w.h = reinterpret_cast<_Float16*>(ws + off);    // n rows, then one row of zeros
  off += up((size_t)(n + 1) * I * 2);
  w.tiles = reinterpret_cast<TileInfo*>(ws + off);
  off += up((size_t)max_tiles * sizeof(TileInfo));
  w.count = reinterpret_cast<int32_t*>(ws + off);
  off += 256;
  w.xexp = reinterpret_cast<int32_t*>(ws + off);
  off += up((size_t)T * 4);
  w.bytes = off;
  return w;
}

template <int BITS, bool YBF16>
moe_status launch_all(const moe_qlayer& q, const BlobLayout& L, const void* x, bool xf32, int T, int k,
                      const int32_t* offsets, const int32_t* sorted_assign, const int32_t* active,
                      const int32_t* n_active, void* y, uint8_t* ws, hipStream_t s) {
  const int n = T * k;
  const int max_active = (int)std::min<int64_t>(q.E, n);
  const int max_tiles = (int)ceil_div(n, kBM) + max_active;
  const MfmaWs W = carve(ws, T, q.H, n, q.E, q.I);

  const int cblocks = std::max(1, std::min(T, 8192));
  uint4* z1 = reinterpret_cast<uint4*>(W.x16 + (size_t)T * q.H);
  uint4* z2 = reinterpret_cast<uint4*>(W.h + (size_t)n * q.I);
  if (xf32)
    to_f16_kernel<true><<<cblocks, 256, 0, s>>>(x, T, q.H / 8, reinterpret_cast<uint4*>(W.x16), W.xexp, z1, q.H / 8,
                                                z2, q.I / 8, W.clip);
  else
    to_f16_kernel<false><<<cblocks, 256, 0, s>>>(x, T, q.H / 8, reinterpret_cast<uint4*>(W.x16), W.xexp, z1, q.H / 8,
                                                 z2, q.I / 8, W.clip);
  if (moe_status st = check_launch("mfma_to_f16")) return st;
  mfma_tiles_kernel<<<1, 1024, 0, s>>>(offsets, active, n_active, q.slot_map, kBM, W.tiles, W.count);
  if (moe_status st = check_launch("mfma_tiles")) return st;

  GemmArgs a;
  a.base = reinterpret_cast<const uint8_t*>(q.base);
  a.stride = q.stride;
  a.H = q.H;
  a.I = q.I;
  a.k = k;
  a.sorted_assign = sorted_assign;
  a.tiles = W.tiles;
  a.tile_count = W.count;
  a.xexp = W.xexp;
  a.clip = W.clip;

  // gate/up: N = 2I in tiles of 64 i values
  a.off_c0 = L.gate_codes;
  a.off_s0 = L.gate_sm;
  a.off_c1 = L.up_codes;
  a.off_s1 = L.up_sm;
  a.a_src = W.x16;
  a.a_zero_row = T;
  a.n_tiles_n = (int)ceil_div(q.I, kBNGateUp / 2);
  a.out = W.h;
  const int tiles_pad = (int)ceil_div(max_tiles, kXcd) * kXcd;  // whole rounds over the dies
  // The pair kernel addresses x, h and an expert blob with 32-bit byte offsets.
  constexpr int64_t kOff = int64_t(1) << 31;
  constexpr bool kPairOk = true;
  const bool off_ok = (int64_t)(T + 1) * q.H * 2 < kOff && (int64_t)(n + 1) * q.I * 2 < kOff && q.stride < kOff;
  // Weights decoded into registers for whole 128-column h tiles and 256-column
  // y tiles.  On the 8,192-token chunk its gate/up took 408, 514 and 470 us
  // for 2-, 3- and 4-bit codes against 519, 594 and 560 for the LDS-decode
  // kernel (one box, Zipf(1.1) routing).
  const bool rb = kRegB && off_ok && q.H % 256 == 0 && q.I % 128 == 0;
  if (rb)
    launch_k(MOE_KERNEL_MFMA_GATEUP, mfma_rb_kernel<BITS, true, false>, dim3((unsigned)(tiles_pad * a.n_tiles_n)),
             dim3(256), 0, s, a);
  else if (kPairOk && off_ok && q.H % 128 == 0)
    launch_k(MOE_KERNEL_MFMA_GATEUP, mfma_ffn_kernel<BITS, kBM, kBNGateUp, true, false, kPairOk, kNT>,
             dim3((unsigned)(tiles_pad * a.n_tiles_n)), dim3(kNT), 0, s, a);
  else
    launch_k(MOE_KERNEL_MFMA_GATEUP, mfma_ffn_kernel<BITS, kBM, kBNGateUp, true, false, false, kNT>,
             dim3((unsigned)(tiles_pad * a.n_tiles_n)), dim3(kNT), 0, s, a);
  if (moe_status st = check_launch("mfma_gateup")) return st;

  // down: N = H in tiles of 128
  a.off_c0 = L.down_codes;
  a.off_s0 = L.down_sm;
  a.a_src = W.h;
  a.a_zero_row = n;
  a.n_tiles_n = (int)ceil_div(q.H, kBNDown);
  a.out = y;
  if (rb)
    launch_k(MOE_KERNEL_MFMA_DOWN, mfma_rb_kernel<BITS, false, YBF16>, dim3((unsigned)(tiles_pad * a.n_tiles_n)),
             dim3(256), 0, s, a);
  else if (kPairOk && off_ok && q.I % 128 == 0)
    launch_k(MOE_KERNEL_MFMA_DOWN, mfma_ffn_kernel<BITS, kBM, kBNDown, false, YBF16, kPairOk, kNT>,
             dim3((unsigned)(tiles_pad * a.n_tiles_n)), dim3(kNT), 0, s, a);
  else
    launch_k(MOE_KERNEL_MFMA_DOWN, mfma_ffn_kernel<BITS, kBM, kBNDown, false, YBF16, false, kNT>,
             dim3((unsigned)(tiles_pad * a.n_tiles_n)), dim3(kNT), 0, s, a);
  return check_launch("mfma_down");
}

}  // namespace

size_t ffn_mfma_ws_bytes(int T, int k, int E, int H, int I) { return carve(nullptr, T, H, T * k, E, I).bytes; }

moe_status launch_ffn_mfma(const moe_qlayer& q, const void* x, moe_dtype x_t, int T, int k, const int32_t* offsets,
                           const int32_t* sorted_assign, const int32_t* active, const int32_t* n_active, void* y,
                           moe_dtype y_t, void* ws, hipStream_t s) {
  const BlobLayout L = blob_layout(q.H, q.I, q.bits);
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  const bool xf = x_t == MOE_F32, yb = y_t == MOE_BF16;
  if (q.bits == 2)
    return yb ? launch_all<2, true>(q, L, x, xf, T, k, offsets, sorted_assign, active, n_active, y, w, s)
              : launch_all<2, false>(q, L, x, xf, T, k, offsets, sorted_assign, active, n_active, y, w, s);
  if (q.bits == 3)
    return yb ? launch_all<3, true>(q, L, x, xf, T, k, offsets, sorted_assign, active, n_active, y, w, s)
              : launch_all<3, false>(q, L, x, xf, T, k, offsets, sorted_assign, active, n_active, y, w, s);
  return yb ? launch_all<4, true>(q, L, x, xf, T, k, offsets, sorted_assign, active, n_active, y, w, s)
            : launch_all<4, false>(q, L, x, xf, T, k, offsets, sorted_assign, active, n_active, y, w, s);
}

}  // namespace moe
