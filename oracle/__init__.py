"""CPU oracle for the MoE expert layer (test infrastructure, not product code).

A plain, slow, fp64 NumPy statement of what the layer computes: FP8 / int4
weight decode, top-k routing, the counting-sort align into padded per-expert
segments with the expert->slot indirection, the per-expert SwiGLU FFN and the
weighted combine. It shares no code with the HIP path and is imported only by
the tests, the smoke check and the benchmark's CPU-baseline leg.

Sources (web pages; cited by title and section):
* "PagedWeight: Efficient MoE LLM Serving with Dynamic Quality-Aware Weight
  Quantization" commentary (spectral-agent.com blog) -- section "what was
  released": an MoE layer runs only a few expert sub-networks per input;
  section "technically interesting points": the router picks experts per
  token and experts are held at a per-expert bit width.
* MOE-GEN explainer (aibr.jp) -- sections 1 and 3: group tokens per expert
  module so each expert sees a large batch.
* "vllm-expert-pager" article (rand.pepabo.com) -- section "hierarchical
  paging of expert weights": per-layer VRAM slots, one expert per slot, and a
  working buffer holding every needed expert when a step needs more experts
  than there are slots; introduction and Table 1 set-up: official FP8 weights
  and the fused w13 (gate+up) / w2 (down) tensors.

Where the pages are silent (softmax and top-k details, SwiGLU, FP8 format,
int4 format, activation quantization) each function states the reading it
takes.
"""
from .numerics import (  # noqa: F401
    E4M3_TABLE, e4m3_decode, e4m3_encode_rne, bf16_decode, f16_decode,
    act_quant_pow2, ACT_GROUP, silu,
)
from .slots import slot_offsets, dequant_slot, FMT_FP8_E4M3_ROW, FMT_INT4_G128  # noqa: F401
from .route import route  # noqa: F401
from .align import align, align_capacity  # noqa: F401
from .ffn import expert_ffn, ACT_BF16, ACT_FP8_G128_POW2  # noqa: F401
from .layer import layer_forward  # noqa: F401
from .router import router_logits, fp32_sum_bound  # noqa: F401
from .requant import bitwidth_plan, requant_slot  # noqa: F401
from .pager import LRUSlots  # noqa: F401
from . import huffman  # noqa: F401
