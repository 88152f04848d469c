"""Float64 CPU oracle for the VDA forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.
"""
from .vda_oracle import *  # noqa: F401,F403
from .vda_oracle import __all__  # noqa: F401
