"""CPU oracle for the MoE layer forward.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (``libmoe.so`` and its binding) never calls it.
"""

from .moe_oracle import *  # noqa: F401,F403
