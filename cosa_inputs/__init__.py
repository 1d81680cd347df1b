"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

Holds workload descriptions and random draws only: no attention, pooling,
scoring or selection arithmetic lives here.
"""
from .configs import HeadPattern, Workload, WORKLOADS, get  # noqa: F401
from .generate import Inputs, make, round_to_bf16  # noqa: F401
