"""MI355X-native MoE token routing on one GPU: router top-k with gate
weights, the expert demand vector, METRO-style greedy replica assignment, the
rank-grouped dispatch layout with single-send dedup counts, row dispatch, an
expert stand-in and the weighted combine, all as hand-written HIP kernels for
gfx950 behind the C ABI in include/moe_route.h.

`binding` mirrors the C entry points one to one; `path` strings them into the
whole path on torch-allocated device buffers. Importing the package loads
libmoe_route.so and fails if it has not been built.
"""
from .binding import (MOE_BF16, MOE_F16, MOE_FLAG_GREEDY_ID_ORDER, MOE_FLAG_OUT_F32,  # noqa: F401
                      MoeError, Problem, make_problem, moe_assign_replicas, moe_combine,
                      moe_combine_backward, moe_dispatch_backward,
                      moe_dispatch, moe_expert_standin, moe_last_error, moe_layout,
                      moe_layout_single_send, moe_route, moe_route_assign_layout,
                      moe_route_assign_layout_noalloc, moe_route_assign_layout_single_send,
                      moe_routing_stats, moe_single_send_dispatch,
                      moe_single_send_expand, moe_status_string, moe_token_balanced_split,
                      moe_version,
                      moe_workspace_bytes)
from . import path  # noqa: F401
