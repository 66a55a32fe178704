"""FP64 CPU oracle of the MoE finalize path (test infrastructure).

Only `tests/`, `__graft_entry__.smoke()` and `bench.py`'s CPU-baseline leg may import this package.
The product path (`moe_expert_output_amd`) never imports it and shares no code with it.
"""
from .moe_finalize_ref import *  # noqa: F401,F403
