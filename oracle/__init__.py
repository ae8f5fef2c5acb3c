"""CPU fp64 oracle of the routed MoE expert computation — TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import or call anything in this package.  The product (the HIP library and its
Python binding) never does, and this package never imports the product.

See ``oracle.moe`` for the definitions and the passages each one follows.
"""
from .moe import (  # noqa: F401
    route, router, router_backward, split_gate_up, merge_gate_up, glu, glu_backward,
    expert_accessor, forward, backward, slot_outputs,
)
