"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU
oracle.  Holds shapes, seeds and random tensors only; no part of the method's
arithmetic."""
from .configs import ALL, BY_INDEX, C1, C2, C3, C4, C5, Workload  # noqa: F401
from . import gen  # noqa: F401
