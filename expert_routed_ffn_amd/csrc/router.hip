// router.hip -- router projection: logits[t][e] = sum_c x[t][c] * Wr[e][c].
//
// Passage: the router scores the experts from a token's hidden state and its
// choice decides which experts run (Strata feature, tech.hub77a.com, section
// "2. 왜 대단한가" (2)).  The pages give no formula; the projection is read as
// a bias-free linear map with bf16 weights Wr [E x H] and fp32 accumulation.
//
// Two kernels:
//   - router_gemv_kernel: one wave per expert row, for up to 16 tokens per
//     workgroup row (decode and verify steps, and fp32 activations).  The
//     weight stream (E * H * 2 bytes) bounds it.  Products and sums in fp32
//     (bf16 times bf16 is exact in fp32).
//   - router_mfma_kernel: bf16 activations and T >= 64 (prefill chunks); a
//     grouped-free GEMM on v_mfma_f32_16x16x32_bf16 with 128 x 128 tiles,
//     K-steps of 32 through double-buffered LDS.  The weight fragment is the
//     first MFMA operand, so a lane holds 4 consecutive experts of one token
//     and stores them as one 16-byte piece.
#include "internal.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---- GEMV -----------------------------------------------------------------

constexpr int kGemvT = 16;  // tokens per workgroup row of the grid

// Grid: (ceil(E / 4), ceil(T / kGemvT)); 256 threads = 4 waves, wave w of
// block b owns expert 4 b + w.  Each lane walks 8-element chunks of the row
// (H % 8 == 0), so the loads of a wave cover 1 KB of the row per step.
template <bool XF32>
__global__ __launch_bounds__(256) void router_gemv_kernel(const void* __restrict__ x, const uint16_t* __restrict__ wr,
                                                          int T, int H, int E, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * kGemvT;
  if (e >= E) return;  // the whole wave leaves
  const int nt = min(kGemvT, T - t0);
  const uint16_t* row = wr + (size_t)e * H;
  float acc[kGemvT];
#pragma unroll
  for (int t = 0; t < kGemvT; ++t) acc[t] = 0.0f;
  // Four 1 KB steps of the row per pass, their loads issued before any use.
  for (int c0 = lane * 8; c0 < H; c0 += 4 * 512) {
    uint4 wv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + 512 * u;
      wv[u] = c < H ? *reinterpret_cast<const uint4*>(row + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + 512 * u;
      if (c >= H) break;
      const float wf[8] = {bf16_lo(wv[u].x), bf16_hi(wv[u].x), bf16_lo(wv[u].y), bf16_hi(wv[u].y),
                           bf16_lo(wv[u].z), bf16_hi(wv[u].z), bf16_lo(wv[u].w), bf16_hi(wv[u].w)};
#pragma unroll
      for (int t = 0; t < kGemvT; ++t) {
        if (t >= nt) continue;  // (a break would keep the loop from unrolling)
        float xf[8];
        const size_t xi = (size_t)(t0 + t) * H + c;
        if constexpr (XF32) {
          const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + xi);
          const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + xi + 4);
          xf[0] = a.x; xf[1] = a.y; xf[2] = a.z; xf[3] = a.w;
          xf[4] = b.x; xf[5] = b.y; xf[6] = b.z; xf[7] = b.w;
        } else {
          const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + xi);
          xf[0] = bf16_lo(v.x); xf[1] = bf16_hi(v.x); xf[2] = bf16_lo(v.y); xf[3] = bf16_hi(v.y);
          xf[4] = bf16_lo(v.z); xf[5] = bf16_hi(v.z); xf[6] = bf16_lo(v.w); xf[7] = bf16_hi(v.w);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[t] = __builtin_fmaf(xf[j], wf[j], acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kGemvT; ++t) {
    if (t >= nt) continue;
    const float v = wave_sum(acc[t]);
    if (lane == 0) logits[(size_t)(t0 + t) * E + e] = v;
  }
}

// ---- MFMA GEMM --------------------------------------------------------------

#ifndef MOE_ROUTER_TM
#define MOE_ROUTER_TM 64
#endif
constexpr int kTileM = MOE_ROUTER_TM;  // tokens per workgroup tile (64: 512 workgroups for 8,192 tokens)
constexpr int kTile = 128;             // experts per workgroup tile
constexpr int kFM = kTileM / 32;       // 16-token fragments per wave
constexpr int kBK = 32;                // K-step: one MFMA's K
static_assert(kTileM == 64 || kTileM == 128, "tokens per router tile");

// 64-byte LDS rows of 32 bf16; 16-byte chunk c of row r sits at c ^ ((r >> 1) & 3)
// (conflict-free for the fragment reads below).
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 32 + ((chunk ^ ((row >> 1) & 3)) * 8); }

// Grid: (ceil(T / kTileM), ceil(E / 128)); 256 threads = 4 waves in a 2 x 2
// grid, each owning kTileM / 2 tokens x 64 experts (kFM x 4 fragments).  Rows
// past T or E read the last valid row and are never stored.  With 64-token
// tiles the 8,192-token chunk runs 512 workgroups, two per CU.
__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr, int T, int H, int E,
                                                          float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_x[2][kTileM * 32];
  __shared__ __attribute__((aligned(16))) uint16_t lds_w[2][kTile * 32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * kTileM, n0 = blockIdx.y * kTile;
  const int KS = H / kBK;

  // loads: thread chunks c = tid and tid + 256: rows r0 = tid / 4 and r0 + 64,
  // 16-byte chunk tid % 4 of each (x takes the second row only for 128-token tiles)
  const int r0 = tid >> 2, r1 = r0 + 64, ch = tid & 3;
  const uint16_t* x0 = x + (size_t)min(m0 + r0, T - 1) * H + ch * 8;
  const uint16_t* x1 = x + (size_t)min(m0 + r1, T - 1) * H + ch * 8;
  const uint16_t* w0 = wr + (size_t)min(n0 + r0, E - 1) * H + ch * 8;
  const uint16_t* w1 = wr + (size_t)min(n0 + r1, E - 1) * H + ch * 8;
  const int o0 = lds_off(r0, ch), o1 = lds_off(r1, ch);
  struct Stage {
    uint4 x0, x1, w0, w1;
  };
  auto load = [&](int ks) {
    const size_t k = (size_t)ks * kBK;
    Stage st;
    st.x0 = *reinterpret_cast<const uint4*>(x0 + k);
    st.x1 = kTileM == 128 ? *reinterpret_cast<const uint4*>(x1 + k) : make_uint4(0, 0, 0, 0);
    st.w0 = *reinterpret_cast<const uint4*>(w0 + k);
    st.w1 = *reinterpret_cast<const uint4*>(w1 + k);
    return st;
  };
  auto store = [&](const Stage st, int buf) {
    *reinterpret_cast<uint4*>(&lds_x[buf][o0]) = st.x0;
    if (kTileM == 128) *reinterpret_cast<uint4*>(&lds_x[buf][o1]) = st.x1;
    *reinterpret_cast<uint4*>(&lds_w[buf][o0]) = st.w0;
    *reinterpret_cast<uint4*>(&lds_w[buf][o1]) = st.w1;
  };

  f32x4_t acc[kFM][4];
#pragma unroll
  for (int fi = 0; fi < kFM; ++fi)
#pragma unroll
    for (int fj = 0; fj < 4; ++fj) acc[fi][fj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fq = lane >> 4;
  auto mma = [&](int buf) {
    bf16x8_t xf[kFM], wf[4];
#pragma unroll
    for (int f = 0; f < kFM; ++f)
      xf[f] = *reinterpret_cast<const bf16x8_t*>(&lds_x[buf][lds_off((kTileM / 2) * wm + 16 * f + fr, fq)]);
#pragma unroll
    for (int f = 0; f < 4; ++f)
      wf[f] = *reinterpret_cast<const bf16x8_t*>(&lds_w[buf][lds_off(64 * wn + 16 * f + fr, fq)]);
#pragma unroll
    for (int fi = 0; fi < kFM; ++fi)
#pragma unroll
      for (int fj = 0; fj < 4; ++fj)
        acc[fi][fj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[fj], xf[fi], acc[fi][fj], 0, 0, 0);
  };

  // Global loads run two K-steps ahead (even stages in s0, odd in s1, from
  // the load to the LDS store); loads past the end repeat the last K-step.
  Stage s0 = load(0), s1 = load(min(1, KS - 1));
  store(s0, 0);
  __syncthreads();
  for (int kb = 0; kb < KS; kb += 2) {
    s0 = load(min(kb + 2, KS - 1));  // s0 held stage kb, already in LDS
    mma(0);
    store(s1, 1);
    __syncthreads();
    if (kb + 1 < KS) {
      s1 = load(min(kb + 3, KS - 1));
      mma(1);
      store(s0, 0);
    }
    __syncthreads();
  }

  // lane: token 16 fi + (lane & 15), experts 16 fj + 4 (lane >> 4) + r
  const bool vec = (E & 3) == 0;
#pragma unroll
  for (int fi = 0; fi < kFM; ++fi) {
    const int t = m0 + (kTileM / 2) * wm + 16 * fi + fr;
    if (t >= T) continue;
    float* out = logits + (size_t)t * E;
#pragma unroll
    for (int fj = 0; fj < 4; ++fj) {
      const int e = n0 + 64 * wn + 16 * fj + 4 * fq;
      const f32x4_t v = acc[fi][fj];
      if (vec && e + 3 < E) {
        *reinterpret_cast<float4*>(out + e) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e + r < E) out[e + r] = v[r];
      }
    }
  }
}

}  // namespace

// bf16 activations with at least this many tokens go to the MFMA kernel.
constexpr int kRouterMfmaMinT = 64;

moe_status launch_router_logits(const void* x, bool xf32, const uint16_t* wr, int T, int H, int E, float* logits,
                                hipStream_t s) {
  if (!xf32 && T >= kRouterMfmaMinT) {
    launch_k(MOE_KERNEL_ROUTER, router_mfma_kernel,
             dim3((unsigned)ceil_div(T, kTileM), (unsigned)ceil_div(E, kTile)), dim3(256), 0, s,
             reinterpret_cast<const uint16_t*>(x), wr, T, H, E, logits);
  } else {
    const dim3 grid((unsigned)ceil_div(E, 4), (unsigned)ceil_div(T, kGemvT));
    if (xf32)
      launch_k(MOE_KERNEL_ROUTER, router_gemv_kernel<true>, grid, dim3(256), 0, s, x, wr, T, H, E, logits);
    else
      launch_k(MOE_KERNEL_ROUTER, router_gemv_kernel<false>, grid, dim3(256), 0, s, x, wr, T, H, E, logits);
  }
  return check_launch("router_logits");
}

}  // namespace moe
