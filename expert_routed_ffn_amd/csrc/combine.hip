// combine.hip -- weighted sum of each token's k expert rows back in token order.
//
// out[t][c] = residual[t][c] + sum_{j=0}^{k-1} w[t][j] * y[t*k + j][c], j ascending,
// in fp32; optionally also the bf16 (round to nearest even) of out, which is
// the next layer's input when layers are chained.  Each thread owns eight
// (H % 8 == 0) or four consecutive columns, so the pass is a plain coalesced
// stream over y.
#include <type_traits>

#include "internal.hpp"

namespace moe {
namespace {

struct F4 {
  float v[4];
};

__device__ __forceinline__ F4 load4(const float* p) {
  const float4 q = *reinterpret_cast<const float4*>(p);
  return {{q.x, q.y, q.z, q.w}};
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ F4 load4(const uint16_t* p) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  return {{bf16_bits_to_f32(q.x & 0xFFFFu), bf16_bits_to_f32(q.x >> 16), bf16_bits_to_f32(q.y & 0xFFFFu),
           bf16_bits_to_f32(q.y >> 16)}};
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

template <typename YT, typename RT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y, const float* __restrict__ w, int T,
                                                      int k, int H, const RT* __restrict__ residual,
                                                      float* __restrict__ out, uint16_t* __restrict__ out_bf16) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  F4 acc = {{0.f, 0.f, 0.f, 0.f}};
  if (residual) acc = load4(residual + (size_t)t * H + c);
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const F4 v = load4(y + ((size_t)t * k + j) * H + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc.v[i] = __builtin_fmaf(wj, v.v[i], acc.v[i]);
  }
  *reinterpret_cast<float4*>(out + (size_t)t * H + c) = make_float4(acc.v[0], acc.v[1], acc.v[2], acc.v[3]);
  if (out_bf16) {
    uint2 b;
    b.x = f32_to_bf16_rne(acc.v[0]) | (f32_to_bf16_rne(acc.v[1]) << 16);
    b.y = f32_to_bf16_rne(acc.v[2]) | (f32_to_bf16_rne(acc.v[3]) << 16);
    *reinterpret_cast<uint2*>(out_bf16 + (size_t)t * H + c) = b;
  }
}

// Eight columns per thread (H % 8 == 0): the k rows' loads are all issued
// before the first multiply-add, which then runs in the same order (j
// ascending from the residual), so the result is bit-identical to the kernel
// above.
struct F8 {
  float v[8];
};
__device__ __forceinline__ F8 load8(const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  return {{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}
// y rows are read once: streaming (nontemporal) loads, which measured 66.4 ->
// 57.9 us on the 8,192-token chunk's bf16 y (335 MB).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ F8 load8_stream(const float* p) {
  const uint4 a = load_stream16(p), b = load_stream16(p + 4);
  return {{__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w),
           __uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z), __uint_as_float(b.w)}};
}
__device__ __forceinline__ F8 load8(const uint16_t* p) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  F8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    r.v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
  return r;
}

template <typename YT, typename RT>
__global__ __launch_bounds__(256) void combine8_kernel(const YT* __restrict__ y, const float* __restrict__ w, int T,
                                                       int k, int H, const RT* __restrict__ residual,
                                                       float* __restrict__ out, uint16_t* __restrict__ out_bf16) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (c >= H) return;
  // raw row bytes stay packed (bf16 rows: 4 registers each) until their turn
  using Raw = typename std::conditional<sizeof(YT) == 2, uint4, F8>::type;
  Raw rows[kMaxK];
  float wj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) {
      const YT* p = y + ((size_t)t * k + j) * H + c;
      if constexpr (sizeof(YT) == 2) rows[j] = load_stream16(p);
      else rows[j] = load8_stream(reinterpret_cast<const float*>(p));
      wj[j] = w[(size_t)t * k + j];
    }
  F8 acc = {{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
  if (residual) acc = load8(residual + (size_t)t * H + c);
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) {
      F8 v;
      if constexpr (sizeof(YT) == 2) {
        const uint32_t q[4] = {rows[j].x, rows[j].y, rows[j].z, rows[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v.v[2 * i] = bf16_bits_to_f32(q[i] & 0xFFFFu);
          v.v[2 * i + 1] = bf16_bits_to_f32(q[i] >> 16);
        }
      } else {
        v = rows[j];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc.v[i] = __builtin_fmaf(wj[j], v.v[i], acc.v[i]);
    }
  float4* o = reinterpret_cast<float4*>(out + (size_t)t * H + c);
  o[0] = make_float4(acc.v[0], acc.v[1], acc.v[2], acc.v[3]);
  o[1] = make_float4(acc.v[4], acc.v[5], acc.v[6], acc.v[7]);
  if (out_bf16) {
    uint4 b;
    b.x = f32_to_bf16_rne(acc.v[0]) | (f32_to_bf16_rne(acc.v[1]) << 16);
    b.y = f32_to_bf16_rne(acc.v[2]) | (f32_to_bf16_rne(acc.v[3]) << 16);
    b.z = f32_to_bf16_rne(acc.v[4]) | (f32_to_bf16_rne(acc.v[5]) << 16);
    b.w = f32_to_bf16_rne(acc.v[6]) | (f32_to_bf16_rne(acc.v[7]) << 16);
    *reinterpret_cast<uint4*>(out_bf16 + (size_t)t * H + c) = b;
  }
}

template <typename YT>
void launch_r(const YT* y, const float* w, int T, int k, int H, const void* residual, moe_dtype r_t, float* out,
              uint16_t* out_bf16, hipStream_t s) {
  if (H % 8 == 0) {
    const dim3 grid8((unsigned)ceil_div(H / 8, 256), (unsigned)T), block8(256);
    if (residual && r_t == MOE_BF16)
      launch_k(MOE_KERNEL_COMBINE, combine8_kernel<YT, uint16_t>, grid8, block8, 0, s, y, w, T, k, H,
               (const uint16_t*)residual, out, out_bf16);
    else
      launch_k(MOE_KERNEL_COMBINE, combine8_kernel<YT, float>, grid8, block8, 0, s, y, w, T, k, H,
               (const float*)residual, out, out_bf16);
    return;
  }
  const dim3 grid((unsigned)ceil_div(H / 4, 256), (unsigned)T), block(256);
  if (residual && r_t == MOE_BF16)
    launch_k(MOE_KERNEL_COMBINE, combine_kernel<YT, uint16_t>, grid, block, 0, s, y, w, T, k, H,
             (const uint16_t*)residual, out, out_bf16);
  else
    launch_k(MOE_KERNEL_COMBINE, combine_kernel<YT, float>, grid, block, 0, s, y, w, T, k, H,
             (const float*)residual, out, out_bf16);
}

}  // namespace

moe_status launch_combine(const void* y, moe_dtype y_t, const float* w, int T, int k, int H, const void* residual,
                          moe_dtype r_t, float* out, uint16_t* out_bf16, hipStream_t s) {
  if (T > 65535) return fail(MOE_EUNSUPPORTED, "moe_combine: T above 65535");
  if (y_t == MOE_BF16)
    launch_r((const uint16_t*)y, w, T, k, H, residual, r_t, out, out_bf16, s);
  else
    launch_r((const float*)y, w, T, k, H, residual, r_t, out, out_bf16, s);
  return check_launch("combine");
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

moe_status launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return MOE_OK;
  const int blocks = (int)std::min<int64_t>(1024, ceil_div(n, 256));
  fill_i32_kernel<<<blocks, 256, 0, s>>>(p, n, v);
  return check_launch("fill_i32");
}

}  // namespace moe
