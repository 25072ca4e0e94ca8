"""MI355X-native Mixture-of-Experts layer forward and backward.

The compute lives in libmoe_dispatch.so (hand-written HIP kernels for
gfx950, C ABI in include/moe_dispatch.h); this package is its thin Python
binding (`_native`), a sequencing helper (`layer.MoELayer`) and the seeded
synthetic workloads (`workloads`).  Importing the package does not load the
library; the first call does, and fails loudly if it has not been built.
"""
from ._native import (  # noqa: F401
    EXPORTED, LIB_PATH, MOE_BF16, MOE_EXPERT_CHOICE, MOE_F32, MOE_GELU, MOE_NSTATS, MOE_SIGMOID,
    MOE_SOFTMAX, MOE_SWIGLU, MOE_TOKEN_CHOICE, STAT_NAMES, MoEError, RouteCfg, RouteMap, lib,
    make_cfg, moe_balance_stats, moe_build_map, moe_combine, moe_dispatch, moe_ec_k, moe_expert_ffn,
    moe_ffn_workspace_size, moe_last_error, moe_max_slots, moe_route_workspace_size, moe_router,
    moe_router_workspace_size, moe_select, moe_status_string, moe_tc_capacity, moe_token_list_len,
    moe_combine_backward, moe_dispatch_backward, moe_expert_ffn_backward, moe_ffn_backward_workspace_size,
    moe_gate_backward, moe_router_backward, moe_router_backward_workspace_size)
