"""Seeded synthetic inputs shared by the GPU tests, the benchmark and the
oracle-side checks.

This package holds input recipes only (random draws, an RMS normalisation of
the drawn Q and K, the TrigFlow-path tangent recipe, row samples).  It contains
none of the attention or attention-derivative arithmetic and imports neither
the oracle nor the library.
"""

from .workloads import (
    WORKLOADS,
    Workload,
    make_inputs,
    sample_rows,
    to_float64,
)

__all__ = ["WORKLOADS", "Workload", "make_inputs", "sample_rows", "to_float64"]
