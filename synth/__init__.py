"""Seeded synthetic workloads (shapes + counter-based generator) shared by the oracle's
tests and the HIP path. Holds none of the decode method's arithmetic."""
from . import configs, gen  # noqa: F401
