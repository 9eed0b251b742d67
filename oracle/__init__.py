"""CPU oracle for the single-GPU MoE routing path: TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in the repository's entry module and the
CPU-baseline leg of the benchmark may import this package. The product path
(the HIP library and its Python binding) never imports, calls or links it, and
it shares no code with that path: both are fed the same seeded inputs from the
separate `synth` package, and nothing else.

The oracle is plain numpy (fp64 where the arithmetic is floating point, except
where the workload fixes fp32) and pure Python for the small sequential parts.
Each function states the passage of the source pages it follows; where the
pages leave a step open, the docstring states the reading taken.

Pin status: every function here is pinned by the CPU tests against something
other than itself (hand-worked examples in tests/golden, closed forms, brute
force on tiny inputs, invariants, or the pages' printed numbers). No function
is "parity unpinned".
"""
from .route import demand_vector, gate_weights, topk_select  # noqa: F401
from .replicas import candidates, greedy_assign, token_balanced_activations  # noqa: F401
from .layout import dedup_counts, expert_ranks, permutation, segment_offsets  # noqa: F401
from .rows import (combine, decode16, dispatch, dispatch_rows, encode16,  # noqa: F401
                   expert_standin)
from .bytes_model import (allgather_bytes_per_gpu, alltoall_bytes_per_gpu,  # noqa: F401
                          crossover_bytes, link_time_s)
from .pipeline import route_and_layout, rows_for  # noqa: F401
from .single_send import (single_send_dispatch, single_send_expand,  # noqa: F401
                          single_send_layout)
from .backward import combine_backward_dw, combine_backward_dy, dispatch_backward  # noqa: F401
from .eplb import (optimal_max_activated, replica_share_index,  # noqa: F401
                   split_tokens_per_gpu, token_balanced_split)
from .stats import (coselection, dirichlet_alpha, gini, routing_stats,  # noqa: F401
                    send_counts, source_ranks, top_pair_coverage)
