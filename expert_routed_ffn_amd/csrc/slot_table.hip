// slot_table.hip -- resident-expert slot table (host side).
#include "internal.hpp"

extern "C" {
moe_status moe_slot_table_create(int, int, int, size_t, const void*, void*, int32_t*, hipStream_t, moe_slot_table**) {
  return moe::fail(MOE_EUNSUPPORTED, "slot table not available in this build");
}
moe_status moe_slot_table_preload(moe_slot_table*, const int32_t*, int, hipStream_t) { return MOE_EUNSUPPORTED; }
moe_status moe_slot_table_resolve(moe_slot_table*, int, const int32_t*, const int32_t*, hipStream_t) {
  return MOE_EUNSUPPORTED;
}
moe_status moe_slot_table_stats(const moe_slot_table*, moe_slot_stats*) { return MOE_EUNSUPPORTED; }
moe_status moe_slot_table_map_host(const moe_slot_table*, int32_t*) { return MOE_EUNSUPPORTED; }
void moe_slot_table_destroy(moe_slot_table*) {}
moe_status moe_slot_table_create_host(int, int, int, moe_copy_fn, void*, moe_slot_table**) { return MOE_EUNSUPPORTED; }
moe_status moe_slot_table_resolve_host(moe_slot_table*, int, const int32_t*, int) { return MOE_EUNSUPPORTED; }
}
