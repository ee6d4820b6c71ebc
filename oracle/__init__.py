"""CPU oracle of the latent-MoE layer forward.

TEST INFRASTRUCTURE ONLY. Only the test suite, the entry point's smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package. The GPU
product path never calls it and shares no code with it.
"""
from .lmoe_oracle import *  # noqa: F401,F403
