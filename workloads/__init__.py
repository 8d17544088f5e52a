"""Synthetic workloads (configs and seeded input generators) for the
owned-partition step.  Shared by the tests and the benchmark."""
from . import configs, gen  # noqa: F401
