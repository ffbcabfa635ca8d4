"""Seeded synthetic inputs for the grouped block-scaled GEMM.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``. This module
only draws and encodes inputs: it holds none of the GEMM's arithmetic, and it
imports neither the oracle nor the library. Both sides consume the same bytes.
"""

from .generate import (  # noqa: F401
    WORKLOADS,
    Problem,
    make_problem,
    quantize_e4m3_rowblocks,
    quantize_e4m3_tiles,
    quantize_mx,
    routing_counts,
)
