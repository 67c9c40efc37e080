"""Routed, low-bit-quantized mixture-of-experts FFN layer for MI355X (gfx950).

The compute lives in libmoe.so (hand-written HIP kernels behind the C ABI in
include/moe.h); this package is its Python binding.
"""
from ._lib import (MOE_BF16, MOE_F32, MOE_OK, Dispatch, ExpertLayer, HostSlotTable, MoeError, SlotTable, abi_version,
                   combine, decode_workspace_bytes, dispatch, expert_bytes, expert_ffn_q, header_functions,
                   layer_decode, layer_decode_noalloc, layer_decode_slots, layer_forward, lib, noalloc_max_bytes,
                   profile_next_launch, route_topk, router_logits, router_topk)

__all__ = ["MOE_BF16", "MOE_F32", "MOE_OK", "Dispatch", "ExpertLayer", "HostSlotTable", "MoeError", "SlotTable",
           "abi_version", "combine", "decode_workspace_bytes", "dispatch", "expert_bytes", "expert_ffn_q",
           "header_functions", "layer_decode", "layer_decode_noalloc", "layer_decode_slots", "layer_forward", "lib",
           "noalloc_max_bytes", "profile_next_launch", "route_topk", "router_logits", "router_topk"]
