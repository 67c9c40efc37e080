// ffn_mfma.hip -- expert FFN for prefill chunks (grouped bf16 MFMA GEMM).
#include "internal.hpp"

namespace moe {

size_t ffn_mfma_ws_bytes(int n_assign, int E, int I) { return (size_t)n_assign * (size_t)I * 2 + (size_t)E * 8 + 4096; }

moe_status launch_ffn_mfma(const moe_qlayer&, const void*, moe_dtype, int, int, const int32_t*, const int32_t*,
                           const int32_t*, const int32_t*, void*, moe_dtype, void*, hipStream_t) {
  return fail(MOE_EUNSUPPORTED, "moe_expert_ffn_q: the MFMA path is not available in this build");
}

}  // namespace moe
