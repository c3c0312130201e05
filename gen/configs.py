"""The five synthetic workloads of the expert layer.

Shapes follow the Qwen-MoE-shaped layers the vllm-expert-pager article serves
(rand.pepabo.com, "vllm-expert-pager"): the 35B-A3B model has 40 MoE layers of
256 experts whose FP8 w13/w2 weights total about 30 GiB (introduction), i.e.
3 MiB per expert = FP8 w13 [1024, 2048] + w2 [2048, 512]; the larger model has
48 layers of 512 experts (section on n-gram table paging).
Per-layer VRAM slot counts (102, 46) are the CACHE_SLOTS values of that
article's Tables 1 and 3. The 16384-token batch stands for MOE-GEN's
module-based batching (aibr.jp explainer, section 3 core technique), which
accumulates many tokens per expert module before running it.
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    Ts: Tuple[int, ...]          # token counts this config is run at
    H: int                       # hidden
    I: int                       # inter (per expert)
    E: int                       # experts per layer
    k: int                       # top-k
    layers: int                  # layers run back to back
    wg_std: float                # router weight std
    zipf: bool                   # add log-Zipf(s=1.1) prior to the logits
    w_std: float = 0.02          # expert weight std
    slots: int = 0               # VRAM slots per layer (0 = all E resident)
    masked_resident: bool = False  # router masked to the resident experts
    int4_frac: float = 0.0       # fraction of experts stored int4-g128
    resident_all_at: int = 1 << 30  # T at or above which all E are resident
    notes: str = field(default="")


CONFIGS = {
    "C0": Config("C0", 0, (16,), 128, 64, 8, 2, 1, 0.1, False,
                 notes="tiny layer, 8-slot pool, permuted slot map"),
    "C1": Config("C1", 1, (1, 8, 32), 2048, 512, 256, 8, 40, 0.05, True,
                 slots=102,
                 notes="decode; 102 slots hold routed + seeded fill"),
    "C2": Config("C2", 2, (16384,), 2048, 512, 256, 8, 1, 0.035, True,
                 notes="module-batched; all 256 resident, identity map"),
    "C3": Config("C3", 3, (32, 4096), 2048, 768, 512, 10, 48, 0.05, True,
                 slots=46, masked_resident=True, resident_all_at=4096,
                 notes="larger experts; T=32 masked to 46 residents"),
    "C4": Config("C4", 4, (8, 8192), 2048, 512, 256, 8, 40, 0.05, True,
                 slots=102, int4_frac=0.3, resident_all_at=8192,
                 notes="mixed FP8 / int4-g128 slots"),
}


def config_by_name(name: str) -> Config:
    return CONFIGS[name]
