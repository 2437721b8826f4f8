"""Seeded synthetic workloads for the DSA sparse-attention decode step.

This package is the only code shared by the CPU oracle and the HIP path.  It
draws random inputs and stores them as raw bytes (bf16 as uint16 bit patterns,
OCP e4m3 as uint8 codes, fp32, int32); it performs none of the method's
arithmetic (no scoring, selection, planning or attention).  The float -> bf16 and
float -> e4m3 casts use torch's own dtype conversions, round-to-nearest-even.
"""
from .configs import CONFIGS, WorkloadSpec, spec
from .gen import make_workload, Workload

__all__ = ["CONFIGS", "WorkloadSpec", "spec", "make_workload", "Workload"]
