"""Float64 CPU oracle for fused linear cross-entropy -- test infrastructure.

Importable only by the tests, the smoke check and the benchmark's CPU-baseline
leg. Nothing in the library imports it.
"""
from .flce_oracle import *  # noqa: F401,F403
from .flce_oracle import __all__  # noqa: F401
