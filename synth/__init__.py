"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke check.

Holds input generation only (random numbers, shapes, bf16 rounding); none of
LoopVQ's arithmetic lives here.
"""
from . import gen, workloads  # noqa: F401
from .workloads import ALL, BY_NAME, Workload  # noqa: F401
