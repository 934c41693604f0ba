"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This package only draws and lays out inputs (queries, paged K/V pools, block tables, free
pool, tags); it contains none of the attention, summary, scoring or compaction arithmetic.
"""
from .configs import Workload, make_workload, WORKLOAD_NAMES, DTYPE_F32, DTYPE_BF16

__all__ = ["Workload", "make_workload", "WORKLOAD_NAMES", "DTYPE_F32", "DTYPE_BF16"]
