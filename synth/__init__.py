"""Seeded synthetic inputs shared by the oracle and the GPU library (no decode arithmetic)."""
from . import workloads  # noqa: F401
