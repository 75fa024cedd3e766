"""MI355X-native MoE decode layer (DeepSeek-V4.1-Flash style): Q2_K/Q3_K
routed experts on raw blocks, bf16 router and shared expert.

The compute lives in libmoe.so (hand-written HIP for gfx950, C ABI declared
in include/moe.h); this package only marshals arguments to it.
"""
from .binding import (MOE_K_DOWN, MOE_K_DOWN2, MOE_K_GATEUP, MOE_K_GATEUP2, MOE_K_READ_PROBE, MOE_K_ROUTER, MOE_K_SHARED_DOWN, MOE_K_SHARED_GU,
                      MOE_SCORE_CR, MOE_SCORE_GLIBC, MOE_SHARED_BF16, MOE_SHARED_KQUANT,
                      MOE_STATUS_BAD_PICK, MOE_STATUS_MISS, MOE_STATUS_NAN_KEY, SCORES_EXP_ONLY, SCORES_EXTENDED, SCORES_GLIBC, Cfg, ExpertCache, Experts, Layer, MoeError,
                      cfg_from_shape, enable_glibc_scores, experts_decode, glibc_score_table, experts_prefill, header_words, layer_forward, layer_forward_noalloc, lib, read_probe,
                      lru_simulate, route_select, scores, scores_host, stack_forward, swiglu_host, time_next_launch,
                      workspace_bytes, workspace_init, workspace_layout)

__all__ = [
    "Cfg", "ExpertCache", "Experts", "Layer", "MoeError", "cfg_from_shape", "enable_glibc_scores", "experts_decode",
    "glibc_score_table", "experts_prefill", "header_words",
    "layer_forward", "layer_forward_noalloc", "lib", "lru_simulate", "read_probe", "route_select", "scores", "scores_host", "stack_forward", "swiglu_host",
    "time_next_launch", "workspace_bytes", "workspace_init", "workspace_layout", "MOE_K_GATEUP", "MOE_K_DOWN",
    "MOE_K_ROUTER", "MOE_K_READ_PROBE", "MOE_K_SHARED_GU", "MOE_K_SHARED_DOWN", "MOE_K_GATEUP2", "MOE_K_DOWN2",
    "MOE_SCORE_CR", "MOE_SCORE_GLIBC", "MOE_SHARED_BF16", "MOE_SHARED_KQUANT", "MOE_STATUS_MISS", "MOE_STATUS_NAN_KEY", "MOE_STATUS_BAD_PICK", "SCORES_EXTENDED", "SCORES_GLIBC", "SCORES_EXP_ONLY",
]
