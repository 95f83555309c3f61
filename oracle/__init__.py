"""CPU oracle of the weight-only-quantized fused MoE layer.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library or its binding.
"""
from .moe_ref import *  # noqa: F401,F403
