// noalloc.hip -- moe_layer_decode for callers that cannot allocate device
// memory: its workspace is a fixed device array of this library.
#include <mutex>

#include "internal.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(1) << 20;  // the largest workspace the variant serves
constexpr int kMaxDevices = 64;

// The decode workspace (h, per-expert descriptors, the routed-row table) of
// every moe_layer_decode_noalloc call on a device.  Every call writes each part
// it reads before reading it, so nothing needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on each device, looked up once per device with
// that device current.  In host code `scratch` names a host-side stand-in, not
// the device array, so only these addresses are passed to kernels.
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

moe_status scratch_ptr(hipStream_t stream, void** out) {
  int cur = 0;
  if (moe_status st = moe::check_hip(hipGetDevice(&cur), "moe_layer_decode_noalloc: hipGetDevice")) return st;
  int dev = cur;
  if (stream != nullptr)
    if (moe_status st = moe::check_hip(hipStreamGetDevice(stream, &dev), "moe_layer_decode_noalloc: hipStreamGetDevice"))
      return st;
  if (dev < 0 || dev >= kMaxDevices) return moe::fail(MOE_EUNSUPPORTED, "moe_layer_decode_noalloc: device index");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    if (dev != cur)
      if (moe_status st = moe::check_hip(hipSetDevice(dev), "moe_layer_decode_noalloc: hipSetDevice")) return st;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (moe_status st = moe::check_hip(e, "moe_layer_decode_noalloc: hipGetSymbolAddress(scratch)")) return st;
    if (!p || reinterpret_cast<uintptr_t>(p) % 256)
      return moe::fail(MOE_EHIP, "moe_layer_decode_noalloc: scratch address missing or misaligned");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_layer_decode_noalloc_max_bytes(void) { return kScratchBytes; }

moe_status moe_layer_decode_noalloc(const moe_qlayer* q, const float* logits, const void* x, moe_dtype x_t, int T,
                                    int k, const void* residual, moe_dtype r_t, int32_t* ids, float* w,
                                    int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, int32_t* active,
                                    int32_t* n_active, void* y, moe_dtype y_t, float* out, uint16_t* out_bf16,
                                    hipStream_t stream) {
  if (!q) return moe::fail(MOE_EINVAL, "moe_layer_decode_noalloc: null moe_qlayer");
  if (T < 0 || k < 1 || q->E < 1) return moe::fail(MOE_EINVAL, "moe_layer_decode_noalloc: T < 0, k < 1 or E < 1");
  const size_t need = moe_layer_decode_workspace_bytes(q, T, k);
  if (need > kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof msg,
             "moe_layer_decode_noalloc: this step needs %zu bytes of workspace, above the fixed %zu-byte scratch "
             "(use moe_layer_decode with a caller workspace)",
             need, kScratchBytes);
    return moe::fail(MOE_EUNSUPPORTED, msg);
  }
  if (T == 0) return moe_layer_decode(q, logits, x, x_t, T, k, residual, r_t, ids, w, offsets, sorted_assign,
                                      assign_pos, active, n_active, y, y_t, out, out_bf16, nullptr, 0, stream);
  void* ws = nullptr;
  if (moe_status st = scratch_ptr(stream, &ws)) return st;
  return moe_layer_decode(q, logits, x, x_t, T, k, residual, r_t, ids, w, offsets, sorted_assign, assign_pos, active,
                          n_active, y, y_t, out, out_bf16, ws, kScratchBytes, stream);
}

}  // extern "C"
