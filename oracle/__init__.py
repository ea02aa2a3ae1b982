"""Plain fp64 CPU oracle for block-wise (Thanos-style) pruning of one linear layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
anything here; only the test suite, the smoke check and the CPU-baseline leg of
the benchmark use it. It shares no code with the HIP library and does not import
it.
"""
from .thanos_oracle import *  # noqa: F401,F403
