"""Oracle package: fp64 CPU definition of the operator.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product library or its binding.
"""
from .gla_oracle import *  # noqa: F401,F403
from .gla_oracle import __all__  # noqa: F401
