"""CPU oracle for the W4A8 progressive-quantized linear layer.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.  The arithmetic lives
in ``w4a8_oracle.c`` (plain C, fp32 / int64); this module builds and loads it
and wraps each step for numpy arrays.
"""
from .oracle import *  # noqa: F401,F403
