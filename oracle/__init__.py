"""CPU float64 oracle of the DSpark draft round.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.
"""
from .dspark_oracle import *  # noqa: F401,F403
