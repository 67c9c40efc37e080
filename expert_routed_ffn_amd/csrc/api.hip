// api.hip -- the C ABI entry points: argument checks, workspace sizes, and
// hand-off to the kernel launchers.  A failing check enqueues nothing.
#include <cstdio>
#include <string>

#include "internal.hpp"

namespace moe {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

moe_status fail(moe_status st, const std::string& msg) {
  set_error(msg);
  return st;
}

moe_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

moe_status check_launch(const char* what) { return check_hip(hipGetLastError(), what); }

ProfileReq& profile_req() {
  static thread_local ProfileReq req;
  return req;
}

static int64_t up256(int64_t v) { return (v + 255) / 256 * 256; }

#ifndef MOE_STAGE_IN_GATEUP
#define MOE_STAGE_IN_GATEUP 1
#endif
constexpr bool kStageInGateup = MOE_STAGE_IN_GATEUP != 0;
#ifndef MOE_RESOLVE_IN_GATEUP
#define MOE_RESOLVE_IN_GATEUP 1
#endif
constexpr bool kResolveInGateup = MOE_RESOLVE_IN_GATEUP != 0;

BlobLayout blob_layout(int H, int I, int bits) {
  const int64_t gu_codes = (int64_t)I * H * bits / 8, gu_sm = (int64_t)I * (H / 32) * 4;
  const int64_t d_codes = (int64_t)H * I * bits / 8, d_sm = (int64_t)H * (I / 32) * 4;
  BlobLayout L;
  int64_t o = 0;
  L.gate_codes = o; o = up256(o + gu_codes);
  L.gate_sm = o;    o = up256(o + gu_sm);
  L.up_codes = o;   o = up256(o + gu_codes);
  L.up_sm = o;      o = up256(o + gu_sm);
  L.down_codes = o; o = up256(o + d_codes);
  L.down_sm = o;    o = up256(o + d_sm);
  L.bytes = o;
  return L;
}

}  // namespace moe

using namespace moe;

namespace {

std::string fmt(const char* f, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  snprintf(buf, sizeof buf, f, a, b, c);
  return buf;
}

moe_status check_ek(const char* fn, int E, int k) {
  if (E < 1 || E > kMaxE) return fail(MOE_EUNSUPPORTED, std::string(fn) + fmt(": E=%lld outside [1, 1024]", E));
  if (k < 1 || k > kMaxK || k > E)
    return fail(MOE_EUNSUPPORTED, std::string(fn) + fmt(": k=%lld outside [1, min(16, E=%lld)]", k, E));
  return MOE_OK;
}

moe_status check_shape(const char* fn, int H, int I, int bits) {
  if (bits < 2 || bits > 4) return fail(MOE_EUNSUPPORTED, std::string(fn) + fmt(": bits=%lld (2, 3 or 4)", bits));
  if (H < 32 || H > 16384 || H % 32)
    return fail(MOE_EUNSUPPORTED, std::string(fn) + fmt(": H=%lld (multiple of 32 in [32, 16384])", H));
  if (I < 32 || I > 8192 || I % 32)
    return fail(MOE_EUNSUPPORTED, std::string(fn) + fmt(": I=%lld (multiple of 32 in [32, 8192])", I));
  return MOE_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_last_error.c_str(); }

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE";
    case MOE_EHIP: return "MOE_EHIP";
    case MOE_ENOTPINNED: return "MOE_ENOTPINNED";
    case MOE_ECAPACITY: return "MOE_ECAPACITY";
  }
  return "unknown moe_status";
}

size_t moe_expert_bytes(int H, int I, int bits) {
  if (check_shape("moe_expert_bytes", H, I, bits) != MOE_OK) return 0;
  return (size_t)blob_layout(H, I, bits).bytes;
}

moe_status moe_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t stream) {
  if (T < 0) return fail(MOE_EINVAL, "moe_route_topk: T < 0");
  if (moe_status st = check_ek("moe_route_topk", E, k)) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !ids || !w) return fail(MOE_EINVAL, "moe_route_topk: null pointer");
  return launch_route_topk(logits, T, E, k, ids, w, stream);
}

moe_status moe_router_logits(const void* x, moe_dtype x_t, const void* w_r, int T, int H, int E, float* logits,
                             hipStream_t stream) {
  if (T < 0) return fail(MOE_EINVAL, "moe_router_logits: T < 0");
  if (x_t != MOE_F32 && x_t != MOE_BF16) return fail(MOE_EINVAL, "moe_router_logits: bad x dtype");
  if (E < 1 || E > kMaxE) return fail(MOE_EUNSUPPORTED, fmt("moe_router_logits: E = %d outside 1..%d", E, kMaxE));
  if (H < 32 || H > 16384 || H % 32 != 0)
    return fail(MOE_EUNSUPPORTED, fmt("moe_router_logits: H = %d (needs a multiple of 32 in 32..16384)", H));
  if (T == 0) return MOE_OK;
  if (!x || !w_r || !logits) return fail(MOE_EINVAL, "moe_router_logits: null pointer");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w_r)) & 15)
    return fail(MOE_EINVAL, "moe_router_logits: x and w_r must be 16-byte aligned");
  return launch_router_logits(x, x_t == MOE_F32, reinterpret_cast<const uint16_t*>(w_r), T, H, E, logits, stream);
}

moe_status moe_router_topk(const void* x, moe_dtype x_t, const void* w_r, int T, int H, int E, int k, float* logits,
                           int32_t* ids, float* w, hipStream_t stream) {
  if (moe_status st = check_ek("moe_router_topk", E, k)) return st;
  if (T > 0 && (!ids || !w)) return fail(MOE_EINVAL, "moe_router_topk: null pointer");
  if (moe_status st = moe_router_logits(x, x_t, w_r, T, H, E, logits, stream)) return st;
  if (T == 0) return MOE_OK;
  return launch_route_topk(logits, T, E, k, ids, w, stream);
}

size_t moe_dispatch_workspace_bytes(int T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  return dispatch_ws_bytes(T * k, E);
}

moe_status moe_dispatch(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* sorted_assign,
                        int32_t* assign_pos, int32_t* active, int32_t* n_active, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  if (T < 0) return fail(MOE_EINVAL, "moe_dispatch: T < 0");
  if (moe_status st = check_ek("moe_dispatch", E, k)) return st;
  if ((int64_t)T * k > (int64_t)1 << 24) return fail(MOE_EUNSUPPORTED, "moe_dispatch: T*k above 2^24");
  if (!offsets || !n_active) return fail(MOE_EINVAL, "moe_dispatch: null pointer");
  if (T > 0 && (!ids || !sorted_assign || !assign_pos || !active))
    return fail(MOE_EINVAL, "moe_dispatch: null pointer");
  const size_t need = dispatch_ws_bytes(T * k, E);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(MOE_EWORKSPACE, fmt("moe_dispatch: workspace %lld bytes, needs %lld", (long long)ws_bytes,
                                    (long long)need));
  return launch_dispatch(ids, T * k, E, offsets, sorted_assign, assign_pos, active, n_active, ws, stream);
}

// AUTO: GEMV up to 128 routed rows, MFMA above.  On the 512-expert, top-10,
// 2048 x 512 layer the two paths cross between T = 12 (GEMV 61 us, MFMA
// 64 us per layer step) and T = 16 (77 us, 67 us).
constexpr int64_t kAutoGemvMaxRows = 128;
static moe_ffn_path resolve_path(moe_ffn_path p, int T, int k) {
  if (p == MOE_PATH_AUTO) return (int64_t)T * k <= kAutoGemvMaxRows ? MOE_PATH_GEMV : MOE_PATH_MFMA;
  return p;
}

size_t moe_expert_ffn_workspace_bytes(const moe_qlayer* q, int T, int k, moe_ffn_path path) {
  if (!q || T < 0 || k < 1) return 0;
  if (resolve_path(path, T, k) == MOE_PATH_GEMV) return ffn_gemv_ws_bytes(T, k, q->E, q->H, q->I);
  return ffn_mfma_ws_bytes(T, k, q->E, q->H, q->I);
}

moe_status moe_expert_ffn_q(const moe_qlayer* q, const void* x, moe_dtype x_t, int T, int k, const int32_t* offsets,
                            const int32_t* sorted_assign, const int32_t* active, const int32_t* n_active, void* y,
                            moe_dtype y_t, moe_ffn_path path, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "moe_expert_ffn_q";
  if (!q) return fail(MOE_EINVAL, "moe_expert_ffn_q: null moe_qlayer");
  if (T < 0) return fail(MOE_EINVAL, "moe_expert_ffn_q: T < 0");
  if (moe_status st = check_ek(fn, q->E, k)) return st;
  if (moe_status st = check_shape(fn, q->H, q->I, q->bits)) return st;
  if (x_t != MOE_F32 && x_t != MOE_BF16) return fail(MOE_EINVAL, "moe_expert_ffn_q: x dtype");
  if (y_t != MOE_F32 && y_t != MOE_BF16) return fail(MOE_EINVAL, "moe_expert_ffn_q: y dtype");
  if (path != MOE_PATH_AUTO && path != MOE_PATH_GEMV && path != MOE_PATH_MFMA)
    return fail(MOE_EINVAL, "moe_expert_ffn_q: path");
  if ((int64_t)T * k > (int64_t)1 << 24) return fail(MOE_EUNSUPPORTED, "moe_expert_ffn_q: T*k above 2^24");
  if (T == 0) return MOE_OK;
  if (!q->base || !x || !offsets || !sorted_assign || !active || !n_active || !y)
    return fail(MOE_EINVAL, "moe_expert_ffn_q: null pointer");
  const int64_t eb = blob_layout(q->H, q->I, q->bits).bytes;
  if (q->stride < eb || q->stride % 256)
    return fail(MOE_EINVAL, fmt("moe_expert_ffn_q: stride %lld (needs >= %lld and a multiple of 256)", q->stride, eb));
  if (!aligned(q->base, 256)) return fail(MOE_EINVAL, "moe_expert_ffn_q: base not 256-byte aligned");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 256))
    return fail(MOE_EINVAL, "moe_expert_ffn_q: x or y not 16-byte aligned, or ws not 256-byte aligned");
  const moe_ffn_path p = resolve_path(path, T, k);
  const size_t need = moe_expert_ffn_workspace_bytes(q, T, k, p);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(MOE_EWORKSPACE, fmt("moe_expert_ffn_q: workspace %lld bytes, needs %lld", (long long)ws_bytes,
                                    (long long)need));
  if (p == MOE_PATH_GEMV)
    return launch_ffn_gemv(*q, x, x_t, T, k, offsets, sorted_assign, active, n_active, y, y_t, ws, stream);
  return launch_ffn_mfma(*q, x, x_t, T, k, offsets, sorted_assign, active, n_active, y, y_t, ws, stream);
}

size_t moe_layer_decode_workspace_bytes(const moe_qlayer* q, int T, int k) {
  if (!q || T < 0 || k < 1 || q->E < 1) return 0;
  return decode_ws(nullptr, T, k, q->E, q->H, q->I).bytes;
}

moe_status moe_layer_decode(const moe_qlayer* q, const float* logits, const void* x, moe_dtype x_t, int T, int k,
                            const void* residual, moe_dtype r_t, int32_t* ids, float* w, int32_t* offsets,
                            int32_t* sorted_assign, int32_t* assign_pos, int32_t* active, int32_t* n_active, void* y,
                            moe_dtype y_t, float* out, uint16_t* out_bf16, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  const char* fn = "moe_layer_decode";
  if (!q) return fail(MOE_EINVAL, "moe_layer_decode: null moe_qlayer");
  if (T < 0) return fail(MOE_EINVAL, "moe_layer_decode: T < 0");
  if (T > kDescT) return fail(MOE_EUNSUPPORTED, fmt("moe_layer_decode: T=%lld above 12", T));
  if (moe_status st = check_ek(fn, q->E, k)) return st;
  if (moe_status st = check_shape(fn, q->H, q->I, q->bits)) return st;
  if (x_t != MOE_F32 && x_t != MOE_BF16) return fail(MOE_EINVAL, "moe_layer_decode: x dtype");
  if (y_t != MOE_F32 && y_t != MOE_BF16) return fail(MOE_EINVAL, "moe_layer_decode: y dtype");
  if (residual && r_t != MOE_F32 && r_t != MOE_BF16) return fail(MOE_EINVAL, "moe_layer_decode: residual dtype");
  if (T == 0) return MOE_OK;
  if (!q->base || !logits || !x || !ids || !w || !offsets || !sorted_assign || !assign_pos || !active || !n_active ||
      !y || !out)
    return fail(MOE_EINVAL, "moe_layer_decode: null pointer");
  const int64_t eb = blob_layout(q->H, q->I, q->bits).bytes;
  if (q->stride < eb || q->stride % 256)
    return fail(MOE_EINVAL, fmt("moe_layer_decode: stride %lld (needs >= %lld and a multiple of 256)", q->stride, eb));
  if (!aligned(q->base, 256)) return fail(MOE_EINVAL, "moe_layer_decode: base not 256-byte aligned");
  const uintptr_t r_align = r_t == MOE_F32 ? 16 : 8;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(out, 16) || !aligned(ws, 256) ||
      (residual && !aligned(residual, r_align)) || (out_bf16 && !aligned(out_bf16, 8)))
    return fail(MOE_EINVAL, "moe_layer_decode: misaligned buffer");
  const DecodeWs W = decode_ws(ws, T, k, q->E, q->H, q->I);
  if (ws_bytes < W.bytes)
    return fail(MOE_EWORKSPACE, fmt("moe_layer_decode: workspace %lld bytes, needs %lld", (long long)ws_bytes,
                                    (long long)W.bytes));
  FoldedCombine fc;
  const bool fold = gemv_folds_combine(q->H, q->I);
  if (fold) {
    fc.w = w;
    fc.residual = residual;
    fc.r_t = r_t;
    fc.out = out;
    fc.out_bf16 = out_bf16;
  }
  if (fold && decode_routes_in_gateup(q->H, q->I, T, k))
    return launch_decode_routed(*q, logits, x, x_t, T, k, ids, w, offsets, sorted_assign, assign_pos, active,
                                n_active, W, y, y_t, fc, stream);
  if (moe_status st = launch_route_dispatch_decode(logits, T, q->E, k, ids, w, offsets, sorted_assign, assign_pos,
                                                   active, n_active, W, stream))
    return st;
  if (moe_status st = launch_ffn_gemv_steps(*q, x, x_t, T, k, sorted_assign, n_active, W, y, y_t, fc, stream))
    return st;
  return fold ? MOE_OK : launch_combine(y, y_t, w, T, k, q->H, residual, r_t, out, out_bf16, stream);
}

moe_status moe_layer_decode_slots(const moe_qlayer* q, moe_slot_table* t, int layer, const float* logits,
                                  const void* x, moe_dtype x_t, int T, int k, const void* residual, moe_dtype r_t,
                                  int32_t* ids, float* w, int32_t* offsets, int32_t* sorted_assign,
                                  int32_t* assign_pos, int32_t* active, int32_t* n_active, void* y, moe_dtype y_t,
                                  float* out, uint16_t* out_bf16, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "moe_layer_decode_slots";
  if (!q) return fail(MOE_EINVAL, "moe_layer_decode_slots: null moe_qlayer");
  if (!slot_table_device_mode(t)) return fail(MOE_EINVAL, "moe_layer_decode_slots: the table is not in device mode");
  const SlotTableView v = slot_table_view(t);
  if (layer < 0 || layer >= v.L) return fail(MOE_EINVAL, "moe_layer_decode_slots: layer out of range");
  if (q->E != v.E || q->base != v.slots || (size_t)q->stride != v.expert_bytes || q->slot_map != v.map + (size_t)layer * v.E)
    return fail(MOE_EINVAL, "moe_layer_decode_slots: q must be the table's view of `layer` (base = slots, stride = "
                            "expert_bytes, slot_map = map + layer * E)");
  if (T < 0) return fail(MOE_EINVAL, "moe_layer_decode_slots: T < 0");
  if (T > kDescT) return fail(MOE_EUNSUPPORTED, fmt("moe_layer_decode_slots: T=%lld above 12", T));
  if (moe_status st = check_ek(fn, q->E, k)) return st;
  if (moe_status st = check_shape(fn, q->H, q->I, q->bits)) return st;
  if ((int64_t)std::min(q->E, T * k) > v.n_slots)
    return fail(MOE_ECAPACITY, "moe_layer_decode_slots: more routed experts possible than slots");
  if (x_t != MOE_F32 && x_t != MOE_BF16) return fail(MOE_EINVAL, "moe_layer_decode_slots: x dtype");
  if (y_t != MOE_F32 && y_t != MOE_BF16) return fail(MOE_EINVAL, "moe_layer_decode_slots: y dtype");
  if (residual && r_t != MOE_F32 && r_t != MOE_BF16) return fail(MOE_EINVAL, "moe_layer_decode_slots: residual dtype");
  if (T == 0) return MOE_OK;
  if (!logits || !x || !ids || !w || !offsets || !sorted_assign || !assign_pos || !active || !n_active || !y || !out)
    return fail(MOE_EINVAL, "moe_layer_decode_slots: null pointer");
  const uintptr_t r_align = r_t == MOE_F32 ? 16 : 8;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(out, 16) || !aligned(ws, 256) ||
      (residual && !aligned(residual, r_align)) || (out_bf16 && !aligned(out_bf16, 8)))
    return fail(MOE_EINVAL, "moe_layer_decode_slots: misaligned buffer");
  const DecodeWs W = decode_ws(ws, T, k, q->E, q->H, q->I);
  if (ws_bytes < W.bytes)
    return fail(MOE_EWORKSPACE, fmt("moe_layer_decode_slots: workspace %lld bytes, needs %lld", (long long)ws_bytes,
                                    (long long)W.bytes));
  if (kResolveInGateup && gemv_stages_misses(q->H, q->I) && decode_routes_in_gateup(q->H, q->I, T, k)) {
    FoldedCombine fc;
    fc.w = w;
    fc.residual = residual;
    fc.r_t = r_t;
    fc.out = out;
    fc.out_bf16 = out_bf16;
    return launch_decode_routed_slots(*q, t, layer, logits, x, x_t, T, k, ids, w, offsets, sorted_assign, assign_pos,
                                      active, n_active, W, y, y_t, fc, stream);
  }
  if (moe_status st = launch_route_dispatch_resolve(logits, T, q->E, k, ids, w, offsets, sorted_assign, assign_pos,
                                                    active, n_active, W, t, layer, stream))
    return st;
  // Wide shapes stage the misses inside the gate/up launch, overlapping their
  // transfer with the resident experts' rows; other shapes copy them first.
  const bool stage = kStageInGateup && gemv_stages_misses(q->H, q->I);
  if (!stage)
    if (moe_status st = launch_slot_copy(t, stream)) return st;
  const MissStage ms{v.copies, v.ncopies, v.host_dev};
  FoldedCombine fc;
  const bool fold = gemv_folds_combine(q->H, q->I);
  if (fold) {
    fc.w = w;
    fc.residual = residual;
    fc.r_t = r_t;
    fc.out = out;
    fc.out_bf16 = out_bf16;
  }
  if (moe_status st = launch_ffn_gemv_steps(*q, x, x_t, T, k, sorted_assign, n_active, W, y, y_t, fc, stream,
                                            stage ? &ms : nullptr))
    return st;
  return fold ? MOE_OK : launch_combine(y, y_t, w, T, k, q->H, residual, r_t, out, out_bf16, stream);
}

moe_status moe_combine(const void* y, moe_dtype y_t, const float* w, int T, int k, int H, const void* residual,
                       moe_dtype r_t, float* out, uint16_t* out_bf16, hipStream_t stream) {
  if (T < 0 || H < 1) return fail(MOE_EINVAL, "moe_combine: T < 0 or H < 1");
  if (k < 1 || k > kMaxK) return fail(MOE_EUNSUPPORTED, "moe_combine: k outside [1, 16]");
  if (H % 4) return fail(MOE_EUNSUPPORTED, "moe_combine: H must be a multiple of 4");
  if (y_t != MOE_F32 && y_t != MOE_BF16) return fail(MOE_EINVAL, "moe_combine: y dtype");
  if (residual && r_t != MOE_F32 && r_t != MOE_BF16) return fail(MOE_EINVAL, "moe_combine: residual dtype");
  if (T == 0) return MOE_OK;
  if (!y || !w || !out) return fail(MOE_EINVAL, "moe_combine: null pointer");
  const uintptr_t r_align = r_t == MOE_F32 ? 16 : 8;
  if (!aligned(y, 16) || !aligned(out, 16) || (residual && !aligned(residual, r_align)) ||
      (out_bf16 && !aligned(out_bf16, 8)))
    return fail(MOE_EINVAL, "moe_combine: misaligned buffer");
  return launch_combine(y, y_t, w, T, k, H, residual, r_t, out, out_bf16, stream);
}

moe_status moe_profile_next_launch(moe_kernel kernel, hipEvent_t start, hipEvent_t stop) {
  if ((int)kernel < 0 || (int)kernel > (int)MOE_KERNEL_ROUTER) return fail(MOE_EINVAL, "moe_profile_next_launch: kernel");
  if (!start || !stop) return fail(MOE_EINVAL, "moe_profile_next_launch: null event");
  ProfileReq& p = profile_req();
  p.kernel = (int)kernel;
  p.start = start;
  p.stop = stop;
  return MOE_OK;
}

}  // extern "C"
