"""FP64 CPU oracle for one Beam MoE block (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package; the product path never imports it.
"""
from .beam_moe_oracle import *  # noqa: F401,F403
