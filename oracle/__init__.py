"""CPU oracle for the MoonEP balanced-dispatch hot path.  TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct numpy implementations of what the hot path
computes: expert counts and maxvio, the redundant-expert plan with its
``cu_seqlens``, per-(token, k) destination rows, the zero-copy permute
(dispatch), the expert SwiGLU FFN forward/backward over the plan's groups, the
gate-weighted unpermute (combine) and the replica gradient reduction
(``reduce_grad``), plus an exact minimum-replica solver used to pin the plan.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP library
(``balanced_token_dispatch_moonep_amd``) and never imports it; the only
common dependency is the seeded input generator in ``workload``.

Floating point is carried in float64.  Every function cites the passage of
the MoonEP pages it follows; where the pages leave a step open the reading
taken is stated at the function.
"""
from .plan import (RoutingError, CapacityError, Plan, validate_routing, expert_counts,
                   maxvio, make_plan, destinations, stats_vector, STAT_NAMES, RULES,
                   ST_BAD_ID, ST_DUP_ID, ST_CAPACITY, ST_OVERFLOW, ST_TRAIN_FALLBACK)
from .layer import (dispatch, combine, groups, prefetch, ffn_forward, ffn_backward,
                    reduce_grad, moe_direct, moe_direct_backward, silu, swiglu_ffn,
                    swiglu_ffn_backward, expert_grad_direct, token_grad_direct)
from .brute import (min_replicas_milp, min_replicas_enum, plan_is_feasible_flow, min_migration_milp,
                    min_migration_enum)
from .memory import buffer_bytes

__all__ = [
    "RoutingError", "CapacityError", "Plan", "validate_routing", "expert_counts", "maxvio",
    "make_plan", "destinations", "stats_vector", "STAT_NAMES", "ST_BAD_ID", "ST_DUP_ID",
    "ST_CAPACITY", "ST_OVERFLOW", "ST_TRAIN_FALLBACK", "dispatch", "combine", "groups",
    "prefetch", "ffn_forward", "ffn_backward", "reduce_grad", "moe_direct",
    "moe_direct_backward", "silu", "swiglu_ffn", "swiglu_ffn_backward", "expert_grad_direct",
    "token_grad_direct", "min_replicas_milp", "min_replicas_enum",
    "plan_is_feasible_flow", "min_migration_milp", "min_migration_enum", "buffer_bytes", "RULES",
]
