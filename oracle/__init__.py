"""CPU oracle of the routed MoE block forward.  TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy code that states what the block computes.  Only the
test suite, the package smoke check and the benchmark's CPU-baseline leg may
import it; the HIP library and its Python binding never do, and the two share
no code.  See ``moe_oracle`` for the steps and ``mxfp8`` for the block format.
"""
from . import mxfp8, moe_oracle  # noqa: F401
from .moe_oracle import forward, forward_tokens  # noqa: F401
