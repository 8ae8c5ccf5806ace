"""Seeded synthetic workloads shared by the tests, the smoke check and the
benchmark.

This package holds the five benchmark configurations and the seeded input
generators.  It contains none of the method's arithmetic: it only draws
Q, K and V (and rounds them to the configuration's element type), so both the
CPU oracle and the HIP path can consume the very same values.
"""

from .configs import WORKLOADS, WorkloadConfig, get_workload
from .generators import make_inputs, round_to_bf16, slice_rngs

__all__ = ["WORKLOADS", "WorkloadConfig", "get_workload", "make_inputs",
           "round_to_bf16", "slice_rngs"]
