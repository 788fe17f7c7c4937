"""Synthetic workloads: parameter-list shapes and seeded input generators.

Holds none of the optimizer's arithmetic; shared by tests, benchmark and smoke check.
"""
from . import shapes, gen  # noqa: F401
