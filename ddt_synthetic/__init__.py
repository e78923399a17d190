"""Seeded synthetic workloads shared by the oracle checks, the GPU tests and the bench.

Holds random draws and sizes only, none of the method's arithmetic.
"""
from . import configs, gen  # noqa: F401
from .configs import Config, CONFIGS, get  # noqa: F401
