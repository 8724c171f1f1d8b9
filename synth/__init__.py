"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the benchmark.

Holds random draws and storage-format casts only; none of the step's arithmetic.
"""
from .configs import CONFIGS, ORDER, get  # noqa: F401
from .gen import Problem, append_inputs, make_problem, query_proj_inputs  # noqa: F401
