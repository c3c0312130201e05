"""MoE expert layer for MI355X (gfx950): route -> align -> paged-slot SwiGLU FFN.

The compute lives in libmoe.so (hand-written HIP, C ABI in include/moe.h);
this package is the thin Python binding over it.
"""
from .binding import (  # noqa: F401
    MoeError, SlotPool, route, route_gemm, align, expert_ffn_pass, SLOT_DEFERRED, Pager, pager_fill, pager_fill_packed, fp8_pack, fp8_unpack, route_align, route_align_workspace_bytes, align_capacity, align_workspace_bytes, expert_ffn,
    ffn_workspace_bytes, dequant_slot, slot_bytes, slot_part_offset, layer, layer_call, layer_call_noalloc, layer_workspace_bytes,
    lib, declared_symbols, quant_act, pool_check, debug_poison, bitwidth_plan, requant_slot,
    LIB_PATH, profile_enable, profile_read, ACT_BF16, ACT_FP8_G128_POW2, FMT_FP8_E4M3_ROW, FMT_INT4_G128,
)
