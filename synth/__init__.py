"""Seeded synthetic inputs for the H2O workloads (shapes, skew, bf16 storage).

Holds no part of the H2O arithmetic; used by the tests, the benchmark and the
smoke check on both sides of the parity comparison."""
from .configs import Workload, WORKLOADS, BY_ID, HEADLINE  # noqa: F401
from . import gen  # noqa: F401
