"""Seeded synthetic attention inputs shared by the tests, the benchmark and the oracle runs.

This package only draws random numbers and lays them out; it holds none of the
operator's arithmetic, so both the HIP path and the CPU oracle can consume the
same inputs without sharing any method code.
"""
from .generators import CONFIGS, WorkloadConfig, config, head_inputs, batch_inputs  # noqa: F401
