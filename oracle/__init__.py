"""CPU oracle for the fused MoE layer with weight-only quantised experts.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never imports, links or calls it, and it imports nothing from
the GPU library.
"""
from .moe_oracle import *  # noqa: F401,F403
