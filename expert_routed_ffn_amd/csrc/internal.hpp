// internal.hpp -- declarations shared by the library's own translation units.
// Nothing here is part of the C ABI (that is include/moe.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "moe.h"

namespace moe {

// Thread-local error text behind moe_last_error().
void set_error(const std::string& msg);
moe_status fail(moe_status st, const std::string& msg);
moe_status check_hip(hipError_t e, const char* what);
// Reports a launch error (hipGetLastError) as MOE_EHIP.
moe_status check_launch(const char* what);

// Byte offsets of the six planes of an expert blob and its size.
struct BlobLayout {
  int64_t gate_codes, gate_sm, up_codes, up_sm, down_codes, down_sm, bytes;
};
BlobLayout blob_layout(int H, int I, int bits);

constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;

// ---- launchers (each returns hipGetLastError()-based status) ---------------

moe_status launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s);

moe_status launch_router_logits(const void* x, bool xf32, const uint16_t* wr, int T, int H, int E, float* logits,
                                hipStream_t s);

size_t dispatch_ws_bytes(int n, int E);
moe_status launch_dispatch(const int32_t* ids, int n, int E, int32_t* offsets, int32_t* sorted_assign,
                           int32_t* assign_pos, int32_t* active, int32_t* n_active, void* ws, hipStream_t s);

// ---- decode path (GEMV) ---------------------------------------------------
// Per active expert: its id, first sorted position, row count and (for the
// first kDescT rows) each row's token and assignment index.  128 bytes.
constexpr int kDescT = 12;
struct SlotDesc {
  int32_t e, p0, ne, pad;
  int32_t tok[kDescT];
  int32_t asg[kDescT];
  int32_t pad2[4];
};
static_assert(sizeof(SlotDesc) == 128, "SlotDesc is one 128-byte record");

// Decode workspace: h [T*k x I] (fp32, or bf16 hi and lo planes in the same
// bytes), the slot descriptors, and per sorted position its (expert,
// assignment) pair with the number of positions.
struct DecodeWs {
  float* h;
  SlotDesc* desc;
  int32_t* rows;   // [T*k][2]
  int32_t* nrows;  // [1]
  int32_t* pos_slot;  // [T*k] slot of each sorted position (decode through a slot table)
  int32_t* record;    // a slot-table resolve outcome (decode through a slot table)
  size_t bytes;
};
DecodeWs decode_ws(void* ws, int T, int k, int E, int H, int I);

size_t ffn_gemv_ws_bytes(int T, int k, int E, int H, int I);
moe_status launch_ffn_gemv(const moe_qlayer& q, const void* x, moe_dtype x_t, int T, int k, const int32_t* offsets,
                           const int32_t* sorted_assign, const int32_t* active, const int32_t* n_active, void* y,
                           moe_dtype y_t, void* ws, hipStream_t s);

// Decode step: route + dispatch + descriptors in one workgroup, then the
// gate/up and down kernels reading the descriptors.
moe_status launch_route_dispatch_decode(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                                        int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos,
                                        int32_t* active, int32_t* n_active, const DecodeWs& W, hipStream_t s);
// The combine folded into the down kernel when `out` is set (wide shapes only;
// returns whether it was folded through *folded).
struct FoldedCombine {
  const float* w = nullptr;
  const void* residual = nullptr;
  moe_dtype r_t = MOE_F32;
  float* out = nullptr;
  uint16_t* out_bf16 = nullptr;
};
bool gemv_folds_combine(int H, int I);

// Decode step in two launches (wide shapes, T*k <= 192): routing inside the
// gate/up launch, then the down kernel with the combine folded in.
bool decode_routes_in_gateup(int H, int I, int T, int k);
moe_status launch_decode_routed(const moe_qlayer& q, const float* logits, const void* x, moe_dtype x_t, int T, int k,
                                int32_t* ids, float* w, int32_t* offsets, int32_t* sorted_assign,
                                int32_t* assign_pos, int32_t* active, int32_t* n_active, const DecodeWs& W, void* y,
                                moe_dtype y_t, const FoldedCombine& fc, hipStream_t s);

// Slot table in device mode (slot_table.hip).
struct SlotDevArgs;
struct SlotTableView {
  int L, E, n_slots;
  size_t expert_bytes;
  const uint8_t* slots;
  const int32_t* map;
  const uint8_t* host_dev;  // device view of the master copy (device mode)
  const int32_t* copies;    // the last device resolve's misses, [2 * n] (slot, l*E + e)
  const int32_t* ncopies;   // [1] n
};
bool slot_table_device_mode(const moe_slot_table* t);
SlotDevArgs slot_dev_args(const moe_slot_table* t);
SlotTableView slot_table_view(const moe_slot_table* t);
moe_status launch_slot_copy(const moe_slot_table* t, hipStream_t stream);
// Decode router followed by the table's resolve of the routed experts, one workgroup (dispatch.hip).
moe_status launch_route_dispatch_resolve(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                                         int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos,
                                         int32_t* active, int32_t* n_active, const DecodeWs& W,
                                         const moe_slot_table* t, int layer, hipStream_t s);

// The misses of a device-mode resolve, staged inside the gate/up launch
// instead of by a copy kernel before it (wide shapes only, see
// gemv_stages_misses): the gate/up rows of a missed expert are read from the
// master copy and written into its slot as they are used, and workgroups at
// the front of the same grid copy the rest of each missed blob.
struct MissStage {
  const int32_t* copies = nullptr;   // [2 * n] (slot, l*E + e) of the resolve's misses
  const int32_t* ncopies = nullptr;  // [1] n
  const uint8_t* host = nullptr;     // device view of the page-locked master copy
};
bool gemv_stages_misses(int H, int I);

// moe_layer_decode_slots for the shapes decode_routes_in_gateup accepts, in two
// launches: gate/up with the routing, the table's resolve (evaluated by every
// workgroup from the state before the launch; the last workgroup to finish
// writes the new state) and the staging of the misses; then down with the
// combine folded in.
moe_status launch_decode_routed_slots(const moe_qlayer& q, const moe_slot_table* t, int layer, const float* logits,
                                      const void* x, moe_dtype x_t, int T, int k, int32_t* ids, float* w,
                                      int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, int32_t* active,
                                      int32_t* n_active, const DecodeWs& W, void* y, moe_dtype y_t,
                                      const FoldedCombine& fc, hipStream_t s);

moe_status launch_ffn_gemv_steps(const moe_qlayer& q, const void* x, moe_dtype x_t, int T, int k,
                                 const int32_t* sorted_assign, const int32_t* n_active, const DecodeWs& W, void* y,
                                 moe_dtype y_t, const FoldedCombine& fc, hipStream_t s,
                                 const MissStage* ms = nullptr);

size_t ffn_mfma_ws_bytes(int T, int k, int E, int H, int I);
moe_status launch_ffn_mfma(const moe_qlayer& q, const void* x, moe_dtype x_t, int T, int k, const int32_t* offsets,
                           const int32_t* sorted_assign, const int32_t* active, const int32_t* n_active, void* y,
                           moe_dtype y_t, void* ws, hipStream_t s);

moe_status launch_combine(const void* y, moe_dtype y_t, const float* w, int T, int k, int H, const void* residual,
                          moe_dtype r_t, float* out, uint16_t* out_bf16, hipStream_t s);

moe_status launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

// Pending timing request of moe_profile_next_launch (per host thread).
struct ProfileReq {
  int kernel = -1;
  hipEvent_t start = nullptr, stop = nullptr;
};
ProfileReq& profile_req();

// Launches `kernel`; when a timing request for kernel id `kid` is pending, the
// launch goes through hipExtLaunchKernelGGL with the requested events.
template <typename F, typename... Args>
inline void launch_k(int kid, F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
  ProfileReq& p = profile_req();
  if (p.kernel == kid) {
    p.kernel = -1;
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, p.start, p.stop, 0, args...);
  } else {
    kernel<<<grid, block, shmem, s>>>(args...);
  }
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
