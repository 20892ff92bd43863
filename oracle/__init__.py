"""fp64 CPU oracle of the ZONOS2 MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, smoke() in __graft_entry__.py
and the CPU-baseline leg of bench.py may import, call or run anything in
this package.  The HIP library never uses it and shares no code,
constant or table with it; the two meet only through the seeded inputs of the
``synth`` package.
"""

from .moe_oracle import (  # noqa: F401
    rmsnorm, router_scores, select_topk, gates, histogram, permutation,
    silu, swiglu_expert, combine, oracle_forward, bias_update, stack_forward, e4m3_value, fp8_weights,
    MARGIN_TOL,
)
