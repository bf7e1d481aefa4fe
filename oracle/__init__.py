"""CPU oracle for fused (residual add ->) RMSNorm -> FP8/FP4 quantization.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's
CPU-baseline leg may use it; the GPU library never does, and the two share no code.
"""
from .oracle import *  # noqa: F401,F403
