"""fp64 CPU oracle of the hybrid layer step.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import this package. The GPU library never calls it and shares no code with it.
"""
from .layer import (  # noqa: F401
    rmsnorm, linear, rope, causal_attention, silu, swiglu, kv_slot_addresses,
    sequence_step, layer_step,
)
