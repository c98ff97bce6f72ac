"""CPU oracle for the int4-expert / int8-router MoE block.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The HIP product path never calls,
links or imports anything here, and this package imports nothing from the HIP
path: the two share only the seeded input generators in `synth`.
"""
from .moe_oracle import *  # noqa: F401,F403
