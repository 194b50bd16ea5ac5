"""Seeded synthetic MLA decode workloads, shared by the tests, the smoke check
and the bench.

This module holds no attention arithmetic: it draws sequence lengths, page
permutations, cache values and queries, encodes them into the cache's byte
formats, and poisons every byte the decode must never read.  Both the GPU
path and the oracle receive identical bytes from here.
"""

from .workloads import (  # noqa: F401
    WorkloadSpec,
    Workload,
    SPECS,
    BENCH_SPEC,
    make_workload,
    quantize_fp8_rows,
    E2M1_MAGNITUDES,
    quantize_fp4_rows,
    fp8_row_stride,
    fp4_row_stride,
    to_torch,
)
