"""CPU oracle for the block top-k sparse-attention decode step.

Test infrastructure only: the tests, the package smoke check and the
benchmark's CPU-baseline leg may use it; the product path never does.
"""
from .vx_oracle import *  # noqa: F401,F403
